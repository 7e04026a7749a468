// NT GEMM on the gfx950 matrix cores: C[M, N] = A[M, K] * W[N, K]^T, both
// operands contiguous along K.  These are the encoder's four weight products
// (QKV, attention output, GeGLU up-projection, down-projection) of the tensai
// "テキスト埋め込み" page, section 何が動くか (encoder paragraph); the int8
// form is the integer matmul of its section 精度と量子化.
//
// One kernel template serves three operand formats.  A K tile is 128 bytes
// of every row whatever the format (32 fp32, 64 bf16 or 128 int8), so the
// data movement is identical:
//
//  * 256 threads, 4 waves in a 2 x 2 grid; a wave owns WM x WN MFMA 16x16
//    output tiles (block tile BM = 32 WM rows by BN = 32 WN columns).
//  * K tiles stream global -> LDS with the gfx950 direct-to-LDS load
//    (global_load_lds_dwordx4: each lane's 16 bytes land in LDS without
//    passing through registers) into a ring of STAGES buffers (STAGES - 1
//    tiles in flight while one is consumed).  Each wave waits for its own
//    oldest loads with s_waitcnt vmcnt(n) and a raw s_barrier publishes
//    them; no fence drains the other tiles in flight.  Small LDS stages
//    leave room for several blocks per CU, which overlap one another's
//    pipeline fill and epilogue.
//  * LDS rows are 128 bytes, unpadded, with the eight 16-byte chunks of row
//    r stored at slot chunk ^ (r & 7): the 8 lanes of a fragment read (rows
//    r..r+7, one chunk) then hit 8 distinct bank groups.
//  * Blocks are ordered so that the blocks one XCD runs (block id mod 8)
//    form a contiguous run of a grouped tile order covering about half of
//    A's rows and a quarter of W's rows, a working set that fits the XCD's
//    4 MB L2 (measured: HBM/MALL fetches fell from 3.4x the operand bytes
//    with a plain n-major order).
//
//   fp32: v_mfma_f32_16x16x4_f32, 4 per 16-k chunk (each lane reads a float4
//         and feeds one element per MFMA; A and W use the same k order).
//   bf16: v_mfma_f32_16x16x32_bf16, one per 32-k chunk, fp32 accumulate.
//   int8: v_mfma_i32_16x16x32_i8, one per 32-k block (exact int32 sum of the
//         block), then acc += float(sum) * w_scale[n, block] in fp32; the
//         block scales of the W tile ride the same LDS ring; the row scale
//         a_scale[m] multiplies once in the epilogue.
//   int4 (weights; activations int8): W rows are 64 bytes of packed codes
//         per 128-input K tile and unpack to int8 in registers before the
//         same MFMA, and acc += float(P) * es per block; a transposed MFMA
//         against all-ones gives the activations' block sums S, and the
//         tile's offset term sum_b S * (-eo) is one fp32 MFMA; the block
//         scales and offsets come from the 16-byte record that rides the
//         LDS ring where the int8 scales do.
//
// Epilogues: STORE (fp32 or bf16), RESID (fp32 C += result), GEGLU.  For
// GEGLU the W tile rows are chosen so that the first half of every wave's
// columns are up-projection rows n (the GELU half) and the second half rows
// I + n (the gate half): the two halves of one output land in the same lane
// and combine in registers, and the [M, 2I] intermediate is never stored.
#include <algorithm>
#include <cmath>
#include <mutex>

#include "common.h"
#include "kernels.h"

#ifndef TTE_BF16_PIPE
#define TTE_BF16_PIPE 1
#endif

namespace tte {

namespace {


template <int PREC>
struct Fmt {
  static constexpr int ES = PREC == P_F32 ? 4 : (PREC == P_BF16 ? 2 : 1);  // A element bytes
};

// Block of WGM x WGN waves; each wave owns WM x WN MFMA 16x16 output tiles.
// A K tile is KT bytes of every operand row (128: 32 fp32, 64 bf16 or 128
// int8; 64 or 256: half or twice that, fp32 and bf16 only), one LDS row
// each.
template <int WM, int WN, int PREC, int STAGES_, int WGM, int WGN, int KT_ = 128>
struct Cfg {
  static constexpr int KT = KT_;
  static constexpr int BK = KT / Fmt<PREC>::ES;  // K elements per tile
  static constexpr int NW = WGM * WGN;  // waves per block
  static constexpr int THREADS = 64 * NW;
  static constexpr int BM = 16 * WM * WGM;
  static constexpr int BN = 16 * WN * WGN;
  static constexpr int ROWS = BM + BN;
  static constexpr bool Q4 = PREC == P_I4;
  static constexpr int WROW = Q4 ? KT / 2 : KT;  // bytes of a W row per K tile (int4: packed codes)
  static constexpr int AREG = BM * KT;           // LDS bytes of the A rows, then the W rows
  static constexpr int WREG = BN * WROW;
  // int8: fp32 scales of 4 blocks per W row; int4: the 16-byte record
  static constexpr int SCALE_BYTES = (PREC == P_I8 || Q4) ? BN * 16 : 0;
  static constexpr int TILE = AREG + WREG + SCALE_BYTES;
  static constexpr int STAGES = STAGES_;
  static constexpr int LDS = STAGES * TILE;
  static constexpr int QA = AREG / 1024;           // 1 KB load instructions of the A rows
  static constexpr int Q = (AREG + WREG) / 1024;   // 1 KB load instructions per K tile
  static constexpr int QW = Q / NW;                // per wave
  static constexpr int PER_TILE = QW + ((PREC == P_I8 || Q4) ? 1 : 0);  // vector-memory ops per wave per tile
  static_assert(AREG % 1024 == 0 && WREG % 1024 == 0 && Q % NW == 0, "tile rows must split evenly over the waves");
  static_assert(QW * NW * 1024 == AREG + WREG, "the load instructions cover the tile exactly");
  static_assert((PREC != P_I8 && !Q4) || BN == 32 * NW, "int8 / int4 scale staging: 32 W rows per wave");
  static_assert(KT == 128 || ((KT == 64 || KT == 256) && PREC != P_I8 && !Q4),
                "K tile of 128 bytes, or 64 / 256 for fp32 / bf16");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

// Row of W that tile row r of n-block nb reads.  GEGLU: in each wave
// column's share of the tile (BN/WGN rows), the first half are GELU-half
// rows n and the second half the matching gate rows N + n.
template <int EPI, int BN, int WGN>
__device__ __forceinline__ int w_row(int r, int nb, int N) {
  if constexpr (EPI == E_GEGLU) {
    constexpr int HW = BN / WGN, QW_ = HW / 2;
    const int wave_col = r / HW, within = r % HW;
    const int base = nb * (BN / 2) + wave_col * QW_;
    return within < QW_ ? base + within : N + base + (within - QW_);
  } else {
    return nb * BN + r;
  }
}

// Issue the direct-to-LDS loads of K tile kt into `stage`: QW 1 KB
// instructions of A/W rows, and for int8 the 16-byte scale vectors of 32 W
// rows (lanes 0..31 of every wave).
template <int QW, int PREC, int KT>
__device__ __forceinline__ void issue_tile(uint8_t* stage, const uint8_t* const* sbase, const uint32_t* soff,
                                           const int* step, const float* s_src, int kt, int wid, int lane,
                                           int scale_at) {
#pragma unroll
  for (int j = 0; j < QW; ++j) dma16(sbase[j] + (soff[j] + (uint32_t)(kt * step[j])), stage + (wid * QW + j) * 1024);
  if constexpr (PREC == P_I8 || PREC == P_I4) {
    if (lane < 32) dma16(s_src + kt * 4, stage + scale_at + wid * 512);
  }
}

// Instruction order for the scheduler over the preceding MFMAs (NM) and
// LDS reads (NR): with MFMA_FIRST one MFMA leads (its operands were read
// earlier), then read / MFMA pairs, then what is left of either; so the
// reads of the next k-step issue between this k-step's MFMAs instead of
// being hoisted ahead of them (which makes the MFMAs wait for every read).
template <int NM, int NR, bool MFMA_FIRST>
__device__ __forceinline__ void interleave() {
  constexpr int lead = MFMA_FIRST ? 1 : 0;
  constexpr int pairs = NR < NM - lead ? NR : NM - lead;
  if constexpr (lead) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
  for (int i = 0; i < pairs; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
  }
  if constexpr (NR > pairs) __builtin_amdgcn_sched_group_barrier(0x100, NR - pairs, 0);
  if constexpr (NM - lead - pairs > 0) __builtin_amdgcn_sched_group_barrier(0x008, NM - lead - pairs, 0);
}

// 8 packed 4-bit codes (4 bytes, the even input in the low nibble) as 8
// int8 values in input order.
__device__ __forceinline__ long unpack_q4(uint32_t x) {
  const uint32_t lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;  // codes 0, 2, 4, 6 / 1, 3, 5, 7
  // v_perm_b32: bytes 0..3 of the second operand are selectors 0..3, of the
  // first 4..7
  const uint32_t a = __builtin_amdgcn_perm(hi, lo, 0x05010400u);  // codes 0, 1, 2, 3
  const uint32_t b = __builtin_amdgcn_perm(hi, lo, 0x07030602u);  // codes 4, 5, 6, 7
  return (long)(((uint64_t)b << 32) | a);
}

// One 4-column chunk of the residual stream x [M, N] as the residual
// epilogue reads and writes it: fp32 (16 bytes), or bf16 (8 bytes; the
// fp32 sum is rounded once, to nearest even).  Rows at or past M read as 0.
template <bool XB>
struct XChunk {
  using type = f32x4;
  __device__ static __forceinline__ f32x4 load(const void* C, int m, int M, int N, int n) {
    return m < M ? *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(C) + (size_t)m * N + n)
                 : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __device__ static __forceinline__ f32x4 widen(f32x4 v) { return v; }
  __device__ static __forceinline__ void store(void* C, int m, int N, int n, f32x4 v) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(C) + (size_t)m * N + n) = v;
  }
};
template <>
struct XChunk<true> {
  using type = u32x2;
  __device__ static __forceinline__ u32x2 load(const void* C, int m, int M, int N, int n) {
    return m < M ? *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(C) + (size_t)m * N + n)
                 : u32x2{0u, 0u};
  }
  __device__ static __forceinline__ f32x4 widen(u32x2 v) {
    return f32x4{__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xFFFF0000u), __uint_as_float(v[1] << 16),
                 __uint_as_float(v[1] & 0xFFFF0000u)};
  }
  __device__ static __forceinline__ void store(void* C, int m, int N, int n, f32x4 v) {
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(C) + (size_t)m * N + n) =
        u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  }
};

template <int PREC, int EPI, int OUT, int WM, int WN, int STAGES, int WGM, int WGN, int KT>
// The 128 x 192 bf16 GeGLU tiles (32 x 96 waves) are held to 4 waves per
// SIMD, 128 registers, so that two blocks share a CU (the compiler spills
// two registers for it); every other shape takes what it needs.
__global__ __launch_bounds__(64 * WGM * WGN) __attribute__((amdgpu_waves_per_eu(WN == 6 && WM == 2 ? 4 : 1))) void k_gemm(const uint8_t* __restrict__ A, const float* __restrict__ a_scale,
                                              const uint8_t* __restrict__ W, const float* __restrict__ w_scale,
                                              void* __restrict__ C, int M, int N, int K, int n_blocks,
                                              int m_blocks, int grp, int splits, QkvOut qo) {
  using F = Fmt<PREC>;
  using G = Cfg<WM, WN, PREC, STAGES, WGM, WGN, KT>;
  constexpr int BM = G::BM, BN = G::BN;
  constexpr int ROW = KT;  // LDS row bytes
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WGN, wn = wid % WGN;
  const int g = lane >> 4, li = lane & 15;

  // XCD-aware tile order: block b runs on XCD b mod 8; XCD x gets a
  // contiguous run of a grouped order (groups of `grp` column blocks, every
  // row block inside a group), so its n_tiles/8 tiles cover about
  // (n_tiles/8)/grp row blocks by grp column blocks of the product; the
  // host picks grp to balance the A rows and W rows that run reads.
  const int n_tiles = n_blocks * m_blocks;
  // split-K: block b computes K part b / n_tiles of tile b % n_tiles
  const int split = blockIdx.x / n_tiles, tile_bid = blockIdx.x - split * n_tiles;
  const int xcd = tile_bid & 7, local = tile_bid >> 3;
  const int per = n_tiles >> 3, extra = n_tiles & 7;
  const int tile = xcd * per + min(xcd, extra) + local;
  const int ng = tile / (m_blocks * grp), gbase = ng * grp, gwidth = min(grp, n_blocks - gbase);
  const int grem = tile - ng * m_blocks * grp;
  const int mb = grem / gwidth, nb = gbase + grem % gwidth;
  const int m0 = mb * BM;
  const size_t row_bytes = (size_t)K * F::ES;
  const int k_part = K / splits;  // elements of K this block reduces over
  const int nk = k_part / G::BK;

  // LDS rows are unpadded and the 16-byte chunk c of row r sits in slot
  // c ^ swizzle(r), so that the rows a fragment read touches (16
  // consecutive rows, one chunk) spread over distinct bank groups:
  //   KT = 256 (16 chunks): swizzle(r) = r & 15;
  //   KT = 128 (8 chunks):  swizzle(r) = r & 7;
  //   KT = 64 (4 chunks):   swizzle(r) = ((i >> 1) ^ (i >> 3)) & 3 with
  //   i = r & 15 (the fragment reads know a row only modulo 16), which
  //   puts any 8 consecutive rows in 8 distinct slots of a 128-byte window
  //   and 16 consecutive rows in 16 distinct slots of 256 bytes.
  // Load plan: instruction j of this wave fills the 1 KB of LDS rows
  // RPI q .. RPI q + RPI - 1 (q = wid * QW + j); lane -> row RPI q + lane /
  // (KT/16), slot lane % (KT/16), which holds chunk slot ^ swizzle(row).
  constexpr int CPRW = KT / 16, RPI = 1024 / KT;  // chunks per row, rows per load instruction
  const int lrow = lane / CPRW, slot = lane % CPRW;
  // int4: the W rows are KT/2 bytes (packed codes) and take the 64-byte
  // row plan (16 rows per instruction, 4-chunk swizzle) after the A rows.
  // Each source is a wave-uniform base (the A rows from the block's first
  // row, or W) plus a 32-bit per-lane byte offset, so the loads take the
  // scalar-base form and a lane keeps one register per instruction.
  const uint8_t* sbase[G::QW];
  uint32_t soff[G::QW];
  int step[G::QW];  // bytes a row advances per K tile
  const int wid_u = __builtin_amdgcn_readfirstlane(wid);
  const uint8_t* a_base = A + (size_t)m0 * row_bytes + (size_t)split * k_part * F::ES;
#pragma unroll
  for (int j = 0; j < G::QW; ++j) {
    const int q = wid_u * G::QW + j;
    if (G::Q4 && q >= G::QA) {
      const int r = 16 * (q - G::QA) + (lane >> 2);  // W row of the tile
      const int i = lane >> 2;  // r & 15
      const int chunk = (lane & 3) ^ (((i >> 1) ^ (i >> 3)) & 3);
      sbase[j] = W + (size_t)split * (k_part / 2);
      soff[j] = (uint32_t)w_row<EPI, BN, WGN>(r, nb, N) * (uint32_t)(K / 2) + chunk * 16;
      step[j] = KT / 2;
      continue;
    }
    const int r = RPI * q + lrow;
    const int chunk = slot ^ (KT == 256 ? (r & 15) : KT == 128 ? (r & 7) : ((((r & 15) >> 1) ^ ((r & 15) >> 3)) & 3));
    if (RPI * q < BM) {  // the instruction's rows are all A rows or all W rows
      sbase[j] = a_base;
      soff[j] = (uint32_t)(min(m0 + r, M - 1) - m0) * (uint32_t)row_bytes + chunk * 16;
    } else {
      sbase[j] = W + (size_t)split * k_part * F::ES;
      soff[j] = (uint32_t)w_row<EPI, BN, WGN>(r - BM, nb, N) * (uint32_t)row_bytes + chunk * 16;
    }
    step[j] = KT;
  }
  // int8 / int4: lanes 0..31 of wave w load the 16 bytes (int8: 4 block
  // scales; int4: the record) of W row 32 w + lane of the tile per K tile.
  const float* s_src = nullptr;
  if constexpr (PREC == P_I8 || PREC == P_I4)
    s_src = w_scale + (size_t)w_row<EPI, BN, WGN>(wid * 32 + (lane & 31), nb, N) * (K / 32) + split * (k_part / 32);

  // bf16 residual products in tiles of at most 8 MFMA tiles per wave (32
  // more registers with fp32 x, 16 with bf16 x; larger wave tiles would
  // spill): the x values this lane adds in the epilogue (its WN 4-column
  // chunks of each of its WM 16-row slabs, in the epilogue's lane order)
  // are loaded before the K loop, so their latency overlaps the loop
  // instead of following it.  No block writes another block's part of x,
  // and the loop's waits for its own (younger) tile loads also cover these.
  constexpr bool XB = EPI == E_RESID && OUT == O_BF16;  // bf16 residual stream
  using XC = typename XChunk<XB>::type;
  constexpr bool XPRE = EPI == E_RESID && PREC == P_BF16 && WM * WN <= 8;
  XC xpre[XPRE ? WM : 1][XPRE ? WN : 1];
  if constexpr (XPRE) {
    constexpr int XCPR = 4 * WN;  // 4-column chunks of a wave's 16 WN columns
    const int n_wave = nb * BN + wn * 16 * WN;
#pragma unroll
    for (int mt = 0; mt < WM; ++mt) {
      const int m_slab = m0 + wm * 16 * WM + mt * 16;
#pragma unroll
      for (int i = 0; i < WN; ++i) {
        const int c = lane + 64 * i, row = c / XCPR, cc = c % XCPR;
        xpre[mt][i] = XChunk<XB>::load(C, m_slab + row, M, N, n_wave + 4 * cc);
      }
    }
    asm volatile("" ::: "memory");  // issued here, ahead of the first K tiles
  }

  f32x4 acc[WM][WN];
#pragma unroll
  for (int a = 0; a < WM; ++a)
#pragma unroll
    for (int b = 0; b < WN; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int swz = KT == 256 ? li : KT == 128 ? (li & 7) : (((li >> 1) ^ (li >> 3)) & 3);
#if TTE_BF16_PIPE
  // (two-stage rings only: with a third stage the later load issue of this
  // scheme measured slower for the long-K down-projection)
  // The residual products (N = hidden, few tiles per pack) run the plain
  // loop below: with four packs in flight the fragment-ahead form was
  // ~1% slower for them, while it stays ahead for the wider products.
  if constexpr (PREC == P_BF16 && G::STAGES == 2 && EPI != E_RESID) {
    // Fragment reads one 32-wide k-step ahead of the MFMAs, across the
    // barrier: the last k-step's MFMAs of tile kt run while the first
    // k-step's fragments of tile kt+1 come from LDS.  The barrier sits
    // after the wave's last fragment read of tile kt has returned, so the
    // stage of tile kt itself is free there and tile kt + STAGES goes into
    // it: the ring holds STAGES tiles in flight (the prologue issues
    // STAGES).
    constexpr int KS = KT / 64;  // 32-element k-steps per tile
    static_assert(KS % 2 == 0, "each tile starts in fragment set 0");
    const int issued0 = min(G::STAGES, nk);
    for (int p = 0; p < issued0; ++p)
      issue_tile<G::QW, PREC, KT>(smem + p * G::TILE, sbase, soff, step, s_src, p, wid, lane, G::AREG + G::WREG);
    wait_vm((issued0 - 1) * G::PER_TILE);  // tile 0 has landed (own loads)
    __builtin_amdgcn_s_barrier();          // ... and every wave's
    asm volatile("" ::: "memory");
    bf16x8 fa[2][WM], fb[2][WN];
    auto read_frags = [&](int stg, int ks, bf16x8* a, bf16x8* b) {
      const uint8_t* st = smem + stg * G::TILE;
      const uint8_t* As = st + (wm * 16 * WM + li) * ROW;
      const uint8_t* Bs = st + G::AREG + (wn * 16 * WN + li) * G::WROW;
      const int off = ((4 * ks + g) ^ swz) << 4;
#pragma unroll
      for (int t = 0; t < WM; ++t) a[t] = *reinterpret_cast<const bf16x8*>(As + t * 16 * ROW + off);
#pragma unroll
      for (int t = 0; t < WN; ++t) b[t] = *reinterpret_cast<const bf16x8*>(Bs + t * 16 * ROW + off);
    };
    auto mfma = [&](const bf16x8* a, const bf16x8* b) {
#pragma unroll
      for (int mt = 0; mt < WM; ++mt)
#pragma unroll
        for (int nt = 0; nt < WN; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt], b[nt], acc[mt][nt], 0, 0, 0);
    };
    read_frags(0, 0, fa[0], fb[0]);
    for (int kt = 0; kt < nk; ++kt) {
      const int stg = kt % G::STAGES;
      // k-steps 0 .. KS-2: the next k-step's fragments are read behind
      // this one's MFMAs (sets alternate; KS is even, so a tile starts in
      // set 0 and its last k-step is in set 1)
#pragma unroll
      for (int ks = 0; ks + 1 < KS; ++ks) {
        mfma(fa[ks & 1], fb[ks & 1]);
        read_frags(stg, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
        interleave<WM * WN, WM + WN, true>();
      }
      // every fragment of tile kt has returned
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      if (kt + 1 < nk) {
        // tile kt + 1 has landed; past the barrier no wave reads stage stg,
        // so tile kt + STAGES goes there
        wait_vm(min(G::STAGES - 2, nk - 2 - kt) * G::PER_TILE);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (kt + G::STAGES < nk)
          issue_tile<G::QW, PREC, KT>(smem + stg * G::TILE, sbase, soff, step, s_src, kt + G::STAGES, wid, lane,
                                      G::AREG + G::WREG);
      }
      // k-step 0 of tile kt + 1 is read behind the last k-step's MFMAs of
      // tile kt (after the last tile the read is of a stage no load writes
      // any more, and unused)
      read_frags((kt + 1) % G::STAGES, 0, fa[0], fb[0]);
      mfma(fa[1], fb[1]);
      interleave<WM * WN, WM + WN, false>();
    }
  } else
#endif
  {
  for (int p = 0; p < G::STAGES - 1 && p < nk; ++p)
    issue_tile<G::QW, PREC, KT>(smem + p * G::TILE, sbase, soff, step, s_src, p, wid, lane, G::AREG + G::WREG);

  for (int kt = 0; kt < nk; ++kt) {
    // this wave's loads of tile kt are done once at most `ahead` tiles of
    // its own loads remain in flight; the barrier publishes every wave's
    const int ahead = min(nk - 1 - kt, G::STAGES - 2);
    wait_vm(ahead * G::PER_TILE);
    __builtin_amdgcn_s_barrier();
    // the stage of tile kt - 1 is free: every wave finished reading it
    if (kt + G::STAGES - 1 < nk)
      issue_tile<G::QW, PREC, KT>(smem + ((kt + G::STAGES - 1) % G::STAGES) * G::TILE, sbase, soff, step, s_src,
                                  kt + G::STAGES - 1, wid, lane, G::AREG + G::WREG);

    const uint8_t* stage = smem + (kt % G::STAGES) * G::TILE;
    const uint8_t* As = stage + (wm * 16 * WM + li) * ROW;
    const uint8_t* Bs = stage + G::AREG + (wn * 16 * WN + li) * G::WROW;

    if constexpr (PREC == P_F32 || PREC == P_BF16) {
#pragma unroll
      for (int cc = 0; cc < KT / 64; ++cc) {
        const int off = ((4 * cc + g) ^ swz) << 4;
        if constexpr (PREC == P_F32) {
          f32x4 af[WM], bf[WN];
#pragma unroll
          for (int t = 0; t < WM; ++t) af[t] = *reinterpret_cast<const f32x4*>(As + t * 16 * ROW + off);
#pragma unroll
          for (int t = 0; t < WN; ++t) bf[t] = *reinterpret_cast<const f32x4*>(Bs + t * 16 * ROW + off);
#pragma unroll
          for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int mt = 0; mt < WM; ++mt)
#pragma unroll
              for (int nt = 0; nt < WN; ++nt)
                acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[mt][s], bf[nt][s], acc[mt][nt], 0, 0, 0);
        } else {
          bf16x8 af[WM], bf[WN];
#pragma unroll
          for (int t = 0; t < WM; ++t) af[t] = *reinterpret_cast<const bf16x8*>(As + t * 16 * ROW + off);
#pragma unroll
          for (int t = 0; t < WN; ++t) bf[t] = *reinterpret_cast<const bf16x8*>(Bs + t * 16 * ROW + off);
#pragma unroll
          for (int mt = 0; mt < WM; ++mt)
#pragma unroll
            for (int nt = 0; nt < WN; ++nt)
              acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mt], bf[nt], acc[mt][nt], 0, 0, 0);
        }
      }
    } else if constexpr (PREC == P_I4) {
      // record of this lane's W row: sc[4], mn[4] (bytes), d, dmin (fp32)
      const uint8_t* rec = stage + G::AREG + G::WREG + 16 * (wn * 16 * WN + li);
      u32x4 rw[WN];
#pragma unroll
      for (int nt = 0; nt < WN; ++nt) rw[nt] = *reinterpret_cast<const u32x4*>(rec + 16 * 16 * nt);
      const int swz4 = ((li >> 1) ^ (li >> 3)) & 3;  // the W rows' 64-byte swizzle (row & 15 = li)
      const long ones = 0x0101010101010101l;
      // s_blk[mt]: the activations' block sum S[row li][block g] of this
      // lane; the all-ones product taken transposed (ones x A^T) leaves
      // S[row li][block c] in every register of the lanes of column li, and
      // the lanes of k-group g keep block c = g
      int s_blk[WM];
#pragma unroll
      for (int mt = 0; mt < WM; ++mt) s_blk[mt] = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int off = (((2 * c + (g >> 1)) ^ swz) << 4) + ((g & 1) << 3);
        long af[WM], bf[WN];
#pragma unroll
        for (int t = 0; t < WM; ++t) af[t] = *reinterpret_cast<const long*>(As + t * 16 * ROW + off);
#pragma unroll
        for (int t = 0; t < WN; ++t)
          bf[t] = unpack_q4(*reinterpret_cast<const uint32_t*>(Bs + t * 16 * G::WROW + ((c ^ swz4) << 4) + 4 * g));
#pragma unroll
        for (int mt = 0; mt < WM; ++mt) {
          const i32x4 st = __builtin_amdgcn_mfma_i32_16x16x32_i8(ones, af[mt], i32x4{0, 0, 0, 0}, 0, 0, 0);
          s_blk[mt] = g == c ? st[0] : s_blk[mt];
#pragma unroll
          for (int nt = 0; nt < WN; ++nt) {
            const float es = __uint_as_float(rw[nt][2]) * (float)((rw[nt][0] >> (8 * c)) & 0xFF);
            const i32x4 p = __builtin_amdgcn_mfma_i32_16x16x32_i8(af[mt], bf[nt], i32x4{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[mt][nt][r] = __builtin_fmaf((float)p[r], es, acc[mt][nt][r]);
          }
        }
      }
      // the offsets of the tile's 4 blocks as one fp32 product:
      // acc[m][n] += sum_b S[m][b] * (-eo[n][b]), with lane (row / column
      // li, block g) holding S[li][g] and -eo[li][g] = -dmin * mn[g]
#pragma unroll
      for (int nt = 0; nt < WN; ++nt) {
        const float neg_eo = -(__uint_as_float(rw[nt][3]) * (float)((rw[nt][1] >> (8 * g)) & 0xFF));
#pragma unroll
        for (int mt = 0; mt < WM; ++mt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32((float)s_blk[mt], neg_eo, acc[mt][nt], 0, 0, 0);
      }
    } else {
      // int8: per 32-input block c, one MFMA per output tile gives the exact
      // int32 block sum P, then acc += float(P) * w_scale[n, c] on the VALU
      // (4 cvt + 4 FMA per MFMA).  Two-block software pipeline: block c + 1's
      // MFMAs go into their own registers while block c's sums are scaled,
      // so the VALU work overlaps the matrix cores instead of waiting for
      // each MFMA's result in turn.  Each accumulator still adds its blocks
      // in order 0 .. 3, as before.
      const float* sc = reinterpret_cast<const float*>(stage + G::AREG + G::WREG);
      f32x4 sw[WN];
#pragma unroll
      for (int nt = 0; nt < WN; ++nt) sw[nt] = *reinterpret_cast<const f32x4*>(sc + 4 * (wn * 16 * WN + nt * 16 + li));
      long af[2][WM], bf[2][WN];
      i32x4 pb[2][WM][WN];
      auto read_blk = [&](int c, long* a, long* b) {
        const int off = (((2 * c + (g >> 1)) ^ swz) << 4) + ((g & 1) << 3);
#pragma unroll
        for (int t = 0; t < WM; ++t) a[t] = *reinterpret_cast<const long*>(As + t * 16 * ROW + off);
#pragma unroll
        for (int t = 0; t < WN; ++t) b[t] = *reinterpret_cast<const long*>(Bs + t * 16 * ROW + off);
      };
      auto mfma_blk = [&](const long* a, const long* b, i32x4 (&pp)[WM][WN]) {
#pragma unroll
        for (int mt = 0; mt < WM; ++mt)
#pragma unroll
          for (int nt = 0; nt < WN; ++nt)
            pp[mt][nt] = __builtin_amdgcn_mfma_i32_16x16x32_i8(a[mt], b[nt], i32x4{0, 0, 0, 0}, 0, 0, 0);
      };
      auto scale_one = [&](const i32x4& pp, f32x4& a, float s_) {
#pragma unroll
        for (int r = 0; r < 4; ++r) a[r] = __builtin_fmaf((float)pp[r], s_, a[r]);
      };
      read_blk(0, af[0], bf[0]);
      mfma_blk(af[0], bf[0], pb[0]);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int cur = c & 1, nxt = cur ^ 1;
        if (c + 1 < 4) {
          read_blk(c + 1, af[nxt], bf[nxt]);
          // pairs (block c + 1's MFMA of tile i, block c's scaling of tile
          // i), kept in this order by scheduling barriers: the VALU reads a
          // sum produced WM * WN MFMAs earlier, so neither unit waits
#pragma unroll
          for (int mt = 0; mt < WM; ++mt)
#pragma unroll
            for (int nt = 0; nt < WN; ++nt) {
              pb[nxt][mt][nt] = __builtin_amdgcn_mfma_i32_16x16x32_i8(af[nxt][mt], bf[nxt][nt], i32x4{0, 0, 0, 0}, 0, 0, 0);
              scale_one(pb[cur][mt][nt], acc[mt][nt], sw[nt][c]);
              __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
          for (int mt = 0; mt < WM; ++mt)
#pragma unroll
            for (int nt = 0; nt < WN; ++nt) scale_one(pb[cur][mt][nt], acc[mt][nt], sw[nt][c]);
        }
      }
    }
  }

  }

  // epilogue: lane holds rows 4g + r of column li in every 16 x 16 tile
  if constexpr (EPI == E_QKV) {
    static_assert(WN == 4, "QKV epilogue: a wave's 64 columns are one head");
    const int n_base = nb * BN + wn * 64;
    constexpr int RBQ = 64 * 4 + 16;
    static_assert(G::NW * 16 * RBQ <= G::LDS, "staging fits the K-tile ring");
    __syncthreads();  // every wave is done with the K-tile ring
    if (n_base < 2 * qo.hidden) {
      // Q or K: the wave's 16-row slabs pass through LDS in fp32 (rows padded
      // by 16 bytes); then lane (row = lane / 4, c = lane % 4) rotates the
      // pairs (d, d + 32) for d = 8c .. 8c + 7 of its row with 16-byte table
      // reads and writes 16-byte vectors of the rotated dims.
      uint8_t* slab = smem + wid * 16 * RBQ;
      const int row = lane >> 2, c = lane & 3;
#pragma unroll
      for (int mt = 0; mt < WM; ++mt) {
        const int m_slab = m0 + wm * 16 * WM + mt * 16;
        float rs[4] = {1.f, 1.f, 1.f, 1.f};
        if constexpr (PREC == P_I8 || PREC == P_I4) {
#pragma unroll
          for (int r = 0; r < 4; ++r) rs[r] = a_scale[min(m_slab + 4 * g + r, M - 1)];
        }
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            *reinterpret_cast<float*>(slab + (4 * g + r) * RBQ + (nt * 16 + li) * 4) = acc[mt][nt][r] * rs[r];
        // LDS operations of one wave complete in order
        __builtin_amdgcn_wave_barrier();
        const int m = m_slab + row;
        if (m < M) {
          const float* xs = reinterpret_cast<const float*>(slab + row * RBQ) + 8 * c;
          const f32x4 x0 = *reinterpret_cast<const f32x4*>(xs), x1 = *reinterpret_cast<const f32x4*>(xs + 4);
          const f32x4 y0 = *reinterpret_cast<const f32x4*>(xs + 32), y1 = *reinterpret_cast<const f32x4*>(xs + 36);
          const int pos = m - qo.seg[m].start;
          const float* ct = qo.cos_tab + pos * 32 + 8 * c;
          const float* st = qo.sin_tab + pos * 32 + 8 * c;
          const f32x4 c0 = *reinterpret_cast<const f32x4*>(ct), c1 = *reinterpret_cast<const f32x4*>(ct + 4);
          const f32x4 s0 = *reinterpret_cast<const f32x4*>(st), s1 = *reinterpret_cast<const f32x4*>(st + 4);
          const f32x4 xr0 = x0 * c0 - y0 * s0, xr1 = x1 * c1 - y1 * s1;
          const f32x4 yr0 = y0 * c0 + x0 * s0, yr1 = y1 * c1 + x1 * s1;
          const size_t at = (size_t)m * N + n_base + 8 * c;
          if constexpr (OUT == O_BF16) {
            const u32x4 px = {pack_bf16x2(xr0[0], xr0[1]), pack_bf16x2(xr0[2], xr0[3]), pack_bf16x2(xr1[0], xr1[1]),
                              pack_bf16x2(xr1[2], xr1[3])};
            const u32x4 py = {pack_bf16x2(yr0[0], yr0[1]), pack_bf16x2(yr0[2], yr0[3]), pack_bf16x2(yr1[0], yr1[1]),
                              pack_bf16x2(yr1[2], yr1[3])};
            *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(C) + at) = px;
            *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(C) + at + 32) = py;
          } else {
            float* cp = reinterpret_cast<float*>(C) + at;
            *reinterpret_cast<f32x4*>(cp) = xr0;
            *reinterpret_cast<f32x4*>(cp + 4) = xr1;
            *reinterpret_cast<f32x4*>(cp + 32) = yr0;
            *reinterpret_cast<f32x4*>(cp + 36) = yr1;
          }
        }
        __builtin_amdgcn_wave_barrier();
      }
    } else {
      // V: transposed, the lane's 4 consecutive tokens of one column at once
#pragma unroll
      for (int mt = 0; mt < WM; ++mt) {
        const int mr = m0 + wm * 16 * WM + mt * 16 + 4 * g;
        float rs[4] = {1.f, 1.f, 1.f, 1.f};
        if constexpr (PREC == P_I8 || PREC == P_I4) {
#pragma unroll
          for (int r = 0; r < 4; ++r) rs[r] = mr + r < M ? a_scale[mr + r] : 0.f;
        }
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          // bf16: the 4 tokens (a multiple of 4 apart from the group start)
          // stay 4 consecutive columns under vt_col_bf16
          const size_t at = (size_t)(n_base - 2 * qo.hidden + nt * 16 + li) * qo.vt_stride +
                            (OUT == O_BF16 ? vt_col_bf16(mr) : mr);
          if constexpr (OUT == O_BF16) {
            uint16_t* vp = reinterpret_cast<uint16_t*>(qo.vt) + at;
            if (mr + 3 < M) {
              // the hardware pack-convert: round to nearest even, as
              // f32_to_bf16 for the finite values here
              const uint32_t lo = pack_bf16x2(acc[mt][nt][0] * rs[0], acc[mt][nt][1] * rs[1]);
              const uint32_t hi = pack_bf16x2(acc[mt][nt][2] * rs[2], acc[mt][nt][3] * rs[3]);
              *reinterpret_cast<uint2*>(vp) = uint2{lo, hi};
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (mr + r < M) vp[r] = f32_to_bf16(acc[mt][nt][r] * rs[r]);
            }
          } else {
            float* vp = reinterpret_cast<float*>(qo.vt) + at;
            if (mr + 3 < M) {
              *reinterpret_cast<f32x4*>(vp) = f32x4{acc[mt][nt][0] * rs[0], acc[mt][nt][1] * rs[1],
                                                    acc[mt][nt][2] * rs[2], acc[mt][nt][3] * rs[3]};
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (mr + r < M) vp[r] = acc[mt][nt][r] * rs[r];
            }
          }
        }
      }
    }
    return;
  }
  // Other epilogues: the wave's results pass through LDS one 16-row slab at
  // a time (row-major, rows padded by 16 bytes so that the 4 row groups of
  // a write land in different banks) and leave as 16-byte vectors of whole
  // rows; the residual form loads all of its 16-byte chunks of a slab, then
  // adds and writes them.
  constexpr bool F32_OUT = EPI == E_RESID || EPI == E_PART || OUT == O_F32;
  constexpr int OES = F32_OUT ? 4 : 2;                     // output element bytes
  constexpr int NT_OUT = EPI == E_GEGLU ? WN / 2 : WN;     // 16-column output tiles per wave
  constexpr int CW = 16 * NT_OUT;                          // output columns per wave
  constexpr int RB = CW * OES + 16;                        // LDS bytes per staged row
  constexpr int CPR = CW * OES / 16;                       // 16-byte chunks per row
  static_assert(G::NW * 16 * RB <= G::LDS, "staging fits the K-tile ring");
  __syncthreads();  // every wave is done with the K-tile ring
  uint8_t* slab = smem + wid * 16 * RB;
  const int n_wave = EPI == E_GEGLU ? nb * (BN / 2) + wn * CW : nb * BN + wn * CW;
#pragma unroll
  for (int mt = 0; mt < WM; ++mt) {
    const int m_slab = m0 + wm * 16 * WM + mt * 16;
    float rs[4] = {1.f, 1.f, 1.f, 1.f};
    if constexpr (PREC == P_I8 || PREC == P_I4) {
#pragma unroll
      for (int r = 0; r < 4; ++r) rs[r] = a_scale[min(m_slab + 4 * g + r, M - 1)];
    }
#pragma unroll
    for (int nt = 0; nt < NT_OUT; ++nt) {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (EPI == E_GEGLU) v[r] = gelu_erf(acc[mt][nt][r] * rs[r]) * (acc[mt][nt + WN / 2][r] * rs[r]);
        else v[r] = acc[mt][nt][r] * rs[r];
      }
      uint8_t* p = slab + (4 * g) * RB + (nt * 16 + li) * OES;
      if constexpr (F32_OUT) {
#pragma unroll
        for (int r = 0; r < 4; ++r) *reinterpret_cast<float*>(p + r * RB) = v[r];
      } else {
        const uint32_t lo = pack_bf16x2(v[0], v[1]), hi = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint16_t*>(p) = (uint16_t)lo;
        *reinterpret_cast<uint16_t*>(p + RB) = (uint16_t)(lo >> 16);
        *reinterpret_cast<uint16_t*>(p + 2 * RB) = (uint16_t)hi;
        *reinterpret_cast<uint16_t*>(p + 3 * RB) = (uint16_t)(hi >> 16);
      }
    }
    // LDS operations of one wave complete in order: the reads below see the
    // writes above, and the next slab's writes follow these reads
    __builtin_amdgcn_wave_barrier();
    if constexpr (EPI == E_RESID) {
      // every load of the slab's rows first, then the stores (the compiler
      // would otherwise wait for each chunk's load behind the previous store)
      constexpr int NI = 16 * CPR / 64;
      static_assert(NI * 64 == 16 * CPR, "whole chunks per lane");
      static_assert(!XPRE || NI == WN, "the prefetched chunks are the epilogue's");
      XC ov[NI];
      f32x4 dv[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int c = lane + 64 * i, row = c / CPR, cc = c % CPR;
        dv[i] = *reinterpret_cast<const f32x4*>(slab + row * RB + cc * 16);
        if constexpr (XPRE) ov[i] = xpre[mt][i];
        else ov[i] = XChunk<XB>::load(C, m_slab + row, M, N, n_wave + 4 * cc);
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int c = lane + 64 * i, row = c / CPR, cc = c % CPR, m = m_slab + row;
        if (m < M) XChunk<XB>::store(C, m, N, n_wave + 4 * cc, XChunk<XB>::widen(ov[i]) + dv[i]);
      }
      __builtin_amdgcn_wave_barrier();
      continue;
    }
#pragma unroll
    for (int c = lane; c < 16 * CPR; c += 64) {
      const int row = c / CPR, cc = c % CPR;
      const int m = m_slab + row;
      if (m >= M) continue;
      const u32x4 d = *reinterpret_cast<const u32x4*>(slab + row * RB + cc * 16);
      const int n = n_wave + cc * (16 / OES);
      if constexpr (EPI == E_PART) {
        *reinterpret_cast<u32x4*>(reinterpret_cast<float*>(C) + ((size_t)split * M + m) * N + n) = d;
      } else {
        *reinterpret_cast<u32x4*>(reinterpret_cast<uint8_t*>(C) + ((size_t)m * N + n) * OES) = d;
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

template <int PREC, int EPI, int OUT, int WM, int WN, int STAGES = 4, int WGM = 2, int WGN = 2, int KT = 128>
void go(const void* A, const float* a_scale, const void* W, const float* w_scale, int M, int N, int K, void* C,
        hipStream_t s, const QkvOut& qo = QkvOut{}, int splits = 1) {
  using G = Cfg<WM, WN, PREC, STAGES, WGM, WGN, KT>;
  // once per instantiation, safe when several host threads launch at once
  static std::once_flag attr_once;
  std::call_once(attr_once, [] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm<PREC, EPI, OUT, WM, WN, STAGES, WGM, WGN, KT>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, G::LDS);
  });
  const int n_blocks = EPI == E_GEGLU ? N / (G::BN / 2) : N / G::BN;
  const int m_blocks = (M + G::BM - 1) / G::BM;
  // group width: an XCD's run of per = tiles/8 tiles reads about
  // (per/grp) BM rows of A and grp BN rows of W; their sum is least at
  // grp = sqrt(per BM / BN)
  const double per = (double)n_blocks * m_blocks / 8.0;
  const int grp = std::max(1, std::min(n_blocks, (int)std::lround(std::sqrt(per * G::BM / G::BN))));
  launch_timed(k_gemm<PREC, EPI, OUT, WM, WN, STAGES, WGM, WGN, KT>, dim3(n_blocks * m_blocks * splits),
               dim3(G::THREADS), G::LDS, s, reinterpret_cast<const uint8_t*>(A), a_scale,
               reinterpret_cast<const uint8_t*>(W), w_scale, C, M, N, K, n_blocks, m_blocks, grp, splits, qo);
}

template <int PREC, int WM, int ST, int WGM = 2, int WGN = 2, int KT = 128, int WN = 4>
void go_prec(int epi, const void* A, const float* a_scale, const void* W, const float* w_scale, int M, int N, int K,
             void* C, int out_kind, hipStream_t s) {
  if (epi == E_RESID) {
    if constexpr (PREC == P_BF16) {
      if (out_kind == O_BF16) {
        go<PREC, E_RESID, O_BF16, WM, WN, ST, WGM, WGN, KT>(A, a_scale, W, w_scale, M, N, K, C, s);
        return;
      }
    }
    go<PREC, E_RESID, O_F32, WM, WN, ST, WGM, WGN, KT>(A, a_scale, W, w_scale, M, N, K, C, s);
  } else if (epi == E_GEGLU) {
    if (out_kind == O_BF16) go<PREC, E_GEGLU, O_BF16, WM, WN, ST, WGM, WGN, KT>(A, a_scale, W, w_scale, M, N, K, C, s);
    else go<PREC, E_GEGLU, O_F32, WM, WN, ST, WGM, WGN, KT>(A, a_scale, W, w_scale, M, N, K, C, s);
  } else {
    if (out_kind == O_BF16) go<PREC, E_STORE, O_BF16, WM, WN, ST, WGM, WGN, KT>(A, a_scale, W, w_scale, M, N, K, C, s);
    else go<PREC, E_STORE, O_F32, WM, WN, ST, WGM, WGN, KT>(A, a_scale, W, w_scale, M, N, K, C, s);
  }
}

// Tile choice, measured on MI355X (bf16, the encoder's shapes at 1.9k and
// 16k tokens; 2 LDS stages of 128-byte K tiles unless noted):
//  * T256: 256 x 256, 8 waves of 128 x 64 (one block per CU): wide products
//    with >= 512 such tiles, and the residual products of >= 8k rows whose
//    width is no multiple of 192;
//  * T256N192: 256 x 192, 8 waves of 128 x 48 (one block per CU): the
//    residual products of >= 8k rows otherwise: 768 columns make 4 tiles
//    a row block instead of 3, so 16k rows fill the 256 CUs exactly
//    (192 blocks of 256 x 256 left 64 idle): 4 texts of 4096 tokens, Wo
//    0.85 -> 0.74 and Wo2 2.23 -> 1.92 ms per pass, 1.418 -> 1.457M
//    tokens/s (interleaved runs);
//  * T128W8 / T192W8: 128 x 128 or 192 x 128, 8 waves of 32 x 64 or
//    48 x 64 (two blocks per CU): every other product (QKV always, GeGLU
//    below the T256 size, the residual products below 8k rows); GeGLU takes
//    128 x 192 (32 x 96 waves) instead of 128 x 128 where that fills one
//    round of 512 blocks.  The
//    height is the one with the smaller ceil(tiles / 256) * rows, a count
//    of tile-rows the busiest CU works through (ties to 192: fewer tiles
//    re-read A less): at 1.9k rows GeGLU runs 803 against 739 TFLOP/s in
//    192-row tiles, at 2048 rows 651 against 771.  For the 768-wide
//    residual products of a ~2k-token pack this leaves most CUs idle when
//    one pack runs alone (90 tiles; 64 x 128 4-wave tiles finish a lone
//    down-projection faster, 30 against 37 us), but packs on concurrent
//    streams fill those CUs and the larger tiles load less per flop: the
//    4-stream pass runs 1.40M against 1.32M tokens/s;
//  * the 4-wave tiles for the 768-wide residual products in fp32, int8 and
//    4-bit (larger tiles measured no faster there: their GEMMs are bound by
//    the VALU block-scale work or the fp32 rate): 32 x 128 when there are
//    few tiles and K is short, else 64 x 128, with a third stage for long
//    K;
//  * int8 (its scale staging feeds 32 W rows per wave) and fp32 (measured
//    slower with 8 waves: GeGLU at 957 tokens 54% against 64% of the fp32
//    peak) keep 4-wave tiles: 128 x 128 once there are >= 1024 such tiles.
enum TileCfg { T32, T64, T64L, T128, T128W8, T192W8, T256, T256N192 };

TileCfg pick_tiles(int prec, int epi, int M, int n_cols, int K) {
  const long tiles128 = (long)((M + 127) / 128) * (n_cols / 128);
  const long tiles256 = (long)((M + 255) / 256) * (n_cols / 256);
  if (prec != P_BF16) {
    if (tiles128 >= 1024) return T128;
  } else {
    if (epi == E_RESID && M >= 8192 && n_cols % 192 == 0) return T256N192;
    if (epi == E_RESID ? (M >= 8192 && n_cols % 256 == 0) : (tiles256 >= 512 && n_cols % 256 == 0)) return T256;
    const long c128 = ((tiles128 + 255) / 256) * 128;
    const long c192 = (((long)((M + 191) / 192) * (n_cols / 128) + 255) / 256) * 192;
    return c192 <= c128 ? T192W8 : T128W8;
  }
  if (tiles128 < 256 && n_cols <= 1024 && K <= 1024) return T32;
  return K > 1024 ? T64L : T64;
}

template <int PREC>
void launch_prec(int epi, const void* A, const float* a_scale, const void* W, const float* w_scale, int M, int N,
                 int K, void* C, int out_kind, hipStream_t s) {
  // Tiles that run a lone product faster measured slower in the pass with
  // packs on four concurrent streams, which shares the chip between them
  // (interleaved runs, tokens/s): residual products in 128 x 64 tiles of 3
  // stages (alone: down-projection 26.0 against 35.0 us) 1.37M against
  // 1.43M, with GeGLU also in 128 x 192 tiles 1.36M, residual in 64 x 64
  // tiles 1.30M.  The 90 large residual blocks of a ~2k-token pack leave
  // most compute units to the other streams' kernels.
  const TileCfg tc = pick_tiles(PREC, epi, M, epi == E_GEGLU ? 2 * N : N, K);
  switch (tc) {
    case T128: go_prec<PREC, 4, 2>(epi, A, a_scale, W, w_scale, M, N, K, C, out_kind, s); break;
    case T32: go_prec<PREC, 1, 2>(epi, A, a_scale, W, w_scale, M, N, K, C, out_kind, s); break;
    case T64L: go_prec<PREC, 2, 3>(epi, A, a_scale, W, w_scale, M, N, K, C, out_kind, s); break;
    case T128W8:
      if constexpr (PREC == P_BF16) {
        // GeGLU: 128 x 192 tiles (8 waves of 32 x 96) where they make one round
        // of 512 blocks (two per CU) and 192 x 128 tiles would not: at 2048
        // rows 512 blocks against 528 (or 768 of 128 x 128), 22.7 against
        // 25.5 us a launch
        const long t192 = (long)((M + 191) / 192) * (2 * N / 128), tn192 = (long)((M + 127) / 128) * (2 * N / 192);
        if (epi == E_GEGLU && (2 * N) % 192 == 0 && t192 > 512 && tn192 <= 512)
          go_prec<PREC, 2, 2, 4, 2, 128, 6>(epi, A, a_scale, W, w_scale, M, N, K, C, out_kind, s);
        else go_prec<PREC, 2, 2, 4, 2>(epi, A, a_scale, W, w_scale, M, N, K, C, out_kind, s);
      }
      break;
    case T192W8:
      if constexpr (PREC == P_BF16) go_prec<PREC, 3, 2, 4, 2>(epi, A, a_scale, W, w_scale, M, N, K, C, out_kind, s);
      break;
    case T256:
      if constexpr (PREC == P_BF16) go_prec<PREC, 8, 2, 2, 4>(epi, A, a_scale, W, w_scale, M, N, K, C, out_kind, s);
      break;
    case T256N192:  // residual products only
      if constexpr (PREC == P_BF16) {
        if (out_kind == O_BF16) go<PREC, E_RESID, O_BF16, 8, 3, 2, 2, 4>(A, a_scale, W, w_scale, M, N, K, C, s);
        else go<PREC, E_RESID, O_F32, 8, 3, 2, 2, 4>(A, a_scale, W, w_scale, M, N, K, C, s);
      }
      break;
    default: go_prec<PREC, 2, 2>(epi, A, a_scale, W, w_scale, M, N, K, C, out_kind, s); break;
  }
}

template <int PREC, int OUT>
void launch_qkv_prec(const void* A, const float* a_scale, const void* W, const float* w_scale, int M, int K,
                     void* qkv, const QkvOut& qo, hipStream_t s, bool fill) {
  const int N = 3 * qo.hidden;
  if (fill && M <= 4096) {
    // a lone caller (the latency mode): 4-wave 64 x 128 tiles, ~540 blocks
    // at 1.9k rows instead of 180 of 192 x 128, which leave 76 CUs idle
    // when no other pack's kernels fill them (QKV 28.8 -> 27.0 ms per
    // single-stream step of 64 packs; with four streams the larger tiles
    // stay ahead)
    go<PREC, E_QKV, OUT, 2, 4, 2>(A, a_scale, W, w_scale, M, N, K, qkv, s, qo);
  } else if constexpr (PREC != P_BF16) {
    if (pick_tiles(PREC, E_QKV, M, N, K) == T128) go<PREC, E_QKV, OUT, 4, 4, 2>(A, a_scale, W, w_scale, M, N, K, qkv, s, qo);
    else go<PREC, E_QKV, OUT, 2, 4, 2>(A, a_scale, W, w_scale, M, N, K, qkv, s, qo);
  } else if (pick_tiles(PREC, E_QKV, M, N, K) == T192W8) {
    go<PREC, E_QKV, OUT, 3, 4, 2, 4, 2>(A, a_scale, W, w_scale, M, N, K, qkv, s, qo);
  } else {
    go<PREC, E_QKV, OUT, 2, 4, 2, 4, 2>(A, a_scale, W, w_scale, M, N, K, qkv, s, qo);
  }
}

}  // namespace


void launch_gemm(int prec, int epi, const void* A, const float* a_scale, const void* W, const float* w_scale, int M,
                 int N, int K, void* C, int out_kind, hipStream_t s) {
  if (M <= 0) return;
  if (prec == P_F32) launch_prec<P_F32>(epi, A, a_scale, W, w_scale, M, N, K, C, out_kind, s);
  else if (prec == P_BF16) launch_prec<P_BF16>(epi, A, a_scale, W, w_scale, M, N, K, C, out_kind, s);
  else if (prec == P_I8) launch_prec<P_I8>(epi, A, a_scale, W, w_scale, M, N, K, C, out_kind, s);
  else launch_prec<P_I4>(epi, A, a_scale, W, w_scale, M, N, K, C, out_kind, s);
}

int residual_splits(int prec, int M, int N, int K, int max_splits) {
  // 96 x 128 tiles of 4 waves take ~56 KB of LDS at two stages, so two
  // blocks share a CU: a product of fewer tiles than the 512 such slots
  // leaves compute units idle, and cutting K into parts fills them.  Each
  // part keeps >= 6 K tiles (the pipeline's fill is paid per part).
  // Measured on MI355X, bf16, back to back: the down-projection of a
  // 1913-token pack (N 768, K 3072) 35.0 us unsplit in 128 x 128 tiles,
  // 18.5 in two parts, 16.3 in three, 14.5 in four; the attention output
  // product (K 768) 7.7 unsplit in 128 x 64 tiles, 7.3 in two parts.
  if (M <= 0 || N % 128 != 0) return 1;
  const int bk = 128 / (prec == P_F32 ? 4 : prec == P_BF16 ? 2 : 1);  // K elements per tile
  if (K % bk != 0) return 1;
  const long tiles = (long)((M + 95) / 96) * (N / 128);
  const int nk = K / bk;
  int best = 1;
  for (int sp = 2; sp <= max_splits; ++sp)
    if (nk % sp == 0 && nk / sp >= 6 && tiles * sp <= 512) best = sp;
  return best;
}

void launch_gemm_splitk(int prec, const void* A, const float* a_scale, const void* W, const float* w_scale, int M,
                        int N, int K, int splits, float* partials, hipStream_t s) {
  if (M <= 0) return;
  // 96 x 128 tiles of 4 waves (48 x 64 each); a third stage when each part
  // is long
  const bool long_k = K / splits > 1024;
  if (prec == P_F32) {
    if (long_k) go<P_F32, E_PART, O_F32, 3, 4, 3>(A, a_scale, W, w_scale, M, N, K, partials, s, QkvOut{}, splits);
    else go<P_F32, E_PART, O_F32, 3, 4, 2>(A, a_scale, W, w_scale, M, N, K, partials, s, QkvOut{}, splits);
  } else if (prec == P_BF16) {
    if (long_k) go<P_BF16, E_PART, O_F32, 3, 4, 3>(A, a_scale, W, w_scale, M, N, K, partials, s, QkvOut{}, splits);
    else go<P_BF16, E_PART, O_F32, 3, 4, 2>(A, a_scale, W, w_scale, M, N, K, partials, s, QkvOut{}, splits);
  } else if (prec == P_I8) {
    if (long_k) go<P_I8, E_PART, O_F32, 3, 4, 3>(A, a_scale, W, w_scale, M, N, K, partials, s, QkvOut{}, splits);
    else go<P_I8, E_PART, O_F32, 3, 4, 2>(A, a_scale, W, w_scale, M, N, K, partials, s, QkvOut{}, splits);
  } else {
    if (long_k) go<P_I4, E_PART, O_F32, 3, 4, 3>(A, a_scale, W, w_scale, M, N, K, partials, s, QkvOut{}, splits);
    else go<P_I4, E_PART, O_F32, 3, 4, 2>(A, a_scale, W, w_scale, M, N, K, partials, s, QkvOut{}, splits);
  }
}

void launch_gemm_qkv(int prec, const void* A, const float* a_scale, const void* W, const float* w_scale, int M, int K,
                     void* qkv, int out_kind, const QkvOut& qo, hipStream_t s, bool fill) {
  if (M <= 0) return;
  if (prec == P_F32) launch_qkv_prec<P_F32, O_F32>(A, a_scale, W, w_scale, M, K, qkv, qo, s, false);
  else if (prec == P_BF16 && out_kind == O_BF16) launch_qkv_prec<P_BF16, O_BF16>(A, a_scale, W, w_scale, M, K, qkv, qo, s, fill);
  else if (prec == P_BF16) launch_qkv_prec<P_BF16, O_F32>(A, a_scale, W, w_scale, M, K, qkv, qo, s, false);
  else if (prec == P_I8) launch_qkv_prec<P_I8, O_F32>(A, a_scale, W, w_scale, M, K, qkv, qo, s, false);
  else launch_qkv_prec<P_I4, O_F32>(A, a_scale, W, w_scale, M, K, qkv, qo, s, false);
}

}  // namespace tte
