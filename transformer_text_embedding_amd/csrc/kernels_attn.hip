// Attention over a pack of texts, one head per block column.
//
// What it computes (tensai "テキスト埋め込み" page, section 何が動くか):
// every token attends to the tokens of its own text in both directions; on
// a global layer to all of them, on a local layer only to those at most
// `window` positions away; RoPE positions restart at 0 in every text
// (packing paragraph), base 160000 on global layers and 10000 on local ones
// (encoder paragraph).  Score = q.k / sqrt(64), softmax over the allowed
// keys, output = sum of p * v.
//
// Inputs come from the QKV projection's epilogue: Q and K already rotated
// (RoPE applied once per token, in fp32, before rounding), V transposed to
// vt[h*64 + d][t].  Texts are contiguous token ranges, so "same text" is
// simply start(q) <= key < end(q); no per-key lookup is needed.
//
// How: flash-style streaming over the packed token axis.  A block takes 64
// consecutive queries (128 on bf16 global layers when the pack's texts
// average >= 1024 tokens: 16 or 32 per wave; they may span several texts) and walks 64-key tiles over the union of their
// allowed key ranges only (a local layer needs at most 64 + 2*window keys, a
// global one the texts of its queries), so fully masked tiles are never
// loaded; a wave also skips the matrix work of tiles outside its own
// queries' range.  K rows and V^T rows of a tile stream
// global -> LDS with direct-to-LDS loads into a double buffer (the next
// tile loads while the current one is used), rows XOR-swizzled by 16-byte
// chunk so fragment reads are conflict-free.
//
// The products are taken transposed, S^T = K Q^T and O^T = V^T P^T, so that
// the matrix-core output layout puts one query per lane column: each lane's
// scores of its query are directly the B operand of the P*V product, and the
// running max / sum / rescale of a query stay in the lanes that hold it.
// Softmax uses exp2 with log2(e)/8 folded into one multiply, against a
// reference max per query that moves only when a score exceeds it by more
// than 8 in log2 units (so P <= 2^8; softmax is unchanged by the reference
// it is taken against): the output and sum are rescaled only on the rare
// tiles where that happens for some lane of the wave.  fp32
// variant: v_mfma_f32_16x16x4_f32; bf16 variant: v_mfma_f32_16x16x32_bf16
// with P rounded to bf16, its per-query sum taken on the matrix cores too
// (against an all-ones block, so numerator and denominator use the same
// rounded P), and all statistics in fp32.
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace tte {

namespace {

constexpr int AKT = 64;  // keys per tile
constexpr float NEG_INF = -__builtin_huge_valf();

// Max / sum over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four 16-lane rows'
// copies of one query column), returned to all four: the gfx950 row-swap
// moves pair rows (0,1), (2,3) and then (01, 23) in registers, with no LDS
// crossbar trip.  Pairs combine in a fixed order (row 0's operand first),
// so every lane gets the same, deterministic value.
__device__ __forceinline__ float rows_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int PREC, int STAGES_ = 2>
struct AttnCfg {
  static constexpr int ES = PREC == P_F32 ? 4 : 2;
  static constexpr int ROWB = 64 * ES;                // bytes of a K row (64 dims) and a V^T row (64 keys)
  static constexpr int TILE = 2 * 64 * ROWB;          // K tile + V^T tile
  static constexpr int STAGES = STAGES_;              // ring of key tiles, STAGES - 1 in flight
  static constexpr int LDS = STAGES * TILE;
  static constexpr int ROWS_PER_Q = 1024 / ROWB;      // rows per 1 KB load instruction
  static constexpr int QW = (2 * 64 / ROWS_PER_Q) / 4;  // load instructions per wave per tile
  // key alignment of a tile's V^T row segment: 16 bytes (fp32), or a whole
  // 32-token group of the bf16 column order (vt_col_bf16)
  static constexpr int ALIGN = PREC == P_F32 ? 4 : 32;
};

template <int PREC, int STAGES, int NQ>
__global__ __launch_bounds__(256) void k_attn(const void* __restrict__ qk, const void* __restrict__ vt, int vt_stride,
                                              void* __restrict__ out, const Seg* __restrict__ seg, int T, int nh,
                                              int is_global, int window, float scale_log2,
                                              const int* __restrict__ off, const int* __restrict__ qunit,
                                              int n_texts) {
  using C = AttnCfg<PREC, STAGES>;
  constexpr int QPW = 16 * NQ;  // queries per wave: NQ 16-query column tiles sharing each K / V^T fragment
  constexpr int BQ = 4 * QPW;   // queries per block
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int H = nh * 64, ld = 3 * H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, li = lane & 15;
  // XCD-aware order: block b of the launch runs on XCD b mod 8, so XCD x
  // takes a contiguous run of the (head, query block) pairs in head-major
  // order; a head's keys and values are then fetched into one or two XCDs'
  // L2 instead of all eight, and neighbouring query blocks (whose local
  // windows share key tiles) meet in the same L2.
  int h, qblk;
  {
    const int nx = gridDim.x, total = nx * gridDim.y;
    const int b = blockIdx.y * nx + blockIdx.x;
    const int xcd = b & 7, local = b >> 3, per = total >> 3, extra = total & 7;
    const int wi = xcd * per + min(xcd, extra) + local;
    h = wi / nx;
    qblk = wi - h * nx;
  }

  // The block's queries [i0, q_end): with qunit, unit qblk of the
  // per-text units of BQ queries (text b owns units qunit[b] ..
  // qunit[b+1] - 1), so a block never spans two texts and walks only its
  // own text's keys; the grid covers an upper bound of the unit count and
  // the blocks past it return at once.  Without, BQ consecutive queries of
  // the pack.
  int i0, q_end;
  if (qunit) {
    const int u = qblk;
    const int lo = wave_find(qunit, n_texts, u);  // the unit's text
    if (lo >= n_texts) return;                     // u is past the last unit
    i0 = off[lo] + BQ * (u - qunit[lo]);
    q_end = min(i0 + BQ, off[lo + 1]);
  } else {
    i0 = qblk * BQ;
    q_end = min(i0 + BQ, T);
  }

  // key range of the block (union over its queries) and of this wave
  const int ilast = q_end - 1;
  const Seg sa = seg[i0], sb = seg[ilast];
  int kstart = sa.start, kend = sb.end;
  if (!is_global) {
    kstart = max(kstart, i0 - window);
    kend = min(kend, ilast + window + 1);
  }
  const int wq0 = i0 + QPW * w;
  const bool wave_any = wq0 < q_end;
  const int wq_lo = min(wq0, q_end - 1), wq_hi = min(wq0 + QPW - 1, q_end - 1);
  const Seg swl = seg[wq_lo], swh = seg[wq_hi];
  int wk_lo = swl.start, wk_hi = swh.end;
  if (!is_global) {
    wk_lo = max(wk_lo, wq_lo - window);
    wk_hi = min(wk_hi, wq_hi + window + 1);
  }

  // this lane's query in each 16-query tile, and the keys it may see:
  // [k_lo, k_lo + k_span) (its text, and on a local layer the window); an
  // invalid query sees none
  int qi[NQ], k_lo[NQ];
  unsigned k_span[NQ];
  f32x4 qf[NQ][4];   // fp32: dims 16 kc + 4 g + e
  bf16x8 qb[NQ][2];  // bf16: dims 32 kc + 8 g + e
#pragma unroll
  for (int qt = 0; qt < NQ; ++qt) {
    qi[qt] = wq0 + 16 * qt + li;
    const bool valid = qi[qt] < q_end;
    const int qrow = valid ? qi[qt] : q_end - 1;
    const Seg qs = seg[qrow];
    int lo = qs.start, hi = qs.end;
    if (!is_global) {
      lo = max(lo, qi[qt] - window);
      hi = min(hi, qi[qt] + window + 1);
    }
    k_lo[qt] = lo;
    k_span[qt] = valid ? (unsigned)(hi - lo) : 0u;
    // Q fragment (already rotated)
    if constexpr (PREC == P_F32) {
      const float* qp = reinterpret_cast<const float*>(qk) + (size_t)qrow * ld + h * 64;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) qf[qt][kc] = *reinterpret_cast<const f32x4*>(qp + 16 * kc + 4 * g);
    } else {
      const uint16_t* qp = reinterpret_cast<const uint16_t*>(qk) + (size_t)qrow * ld + h * 64;
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) qb[qt][kc] = *reinterpret_cast<const bf16x8*>(qp + 32 * kc + 8 * g);
    }
  }

  // ---- load plan: instruction j of wave w (q = w * QW + j) fills tile
  // rows ROWS_PER_Q * q .. + ROWS_PER_Q - 1: K rows while ROWS_PER_Q * q <
  // 64 (a wave-uniform test), V^T rows (dims) after.  Each source is a
  // wave-uniform base that advances by one tile of keys per tile plus a
  // per-lane 32-bit offset fixed before the loop, so a tile's loads take no
  // vector address arithmetic; only a K tile running past the pack's last
  // token clamps its rows (V^T has 64 columns of slack). ----
  constexpr int CPR = C::ROWB / 16;  // 16-byte chunks per row
  const int j_first = kstart & ~(C::ALIGN - 1);
  const int n_tiles = (kend - j_first + AKT - 1) / AKT;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int lrow = lane / CPR, lslot = lane % CPR;
  const uint32_t k_row_bytes = (uint32_t)ld * C::ES;
  const uint8_t* k_base = reinterpret_cast<const uint8_t*>(qk) + (size_t)(H + h * 64) * C::ES;
  const uint8_t* v_base = reinterpret_cast<const uint8_t*>(vt) + ((size_t)(h * 64) * vt_stride + j_first) * C::ES;
  // the 32-bit offsets cover every source byte of the pack (else the
  // tiles take the 64-bit form below)
  const bool off32 = (size_t)(T + AKT) * k_row_bytes < ((size_t)1 << 32) &&
                     (size_t)H * (size_t)vt_stride * C::ES < ((size_t)1 << 32);
  uint32_t src_off[C::QW];
#pragma unroll
  for (int j = 0; j < C::QW; ++j) {
    const int q = wu * C::QW + j;
    const int row = C::ROWS_PER_Q * q + lrow;
    const uint32_t chunk = (uint32_t)((lslot ^ (row & 7)) * 16);
    src_off[j] = C::ROWS_PER_Q * q < 64 ? (uint32_t)(j_first + row) * k_row_bytes + chunk
                                        : (uint32_t)(row - 64) * (uint32_t)vt_stride * C::ES + chunk;
  }
  auto issue = [&](int t) {
    uint8_t* stage = smem + (t % C::STAGES) * C::TILE;
    // every K row of the tile is a token of the pack
    if (off32 && j_first + (t + 1) * AKT <= T) {
      // the wave's loads are all K rows or all V^T rows
      static_assert(64 % (C::QW * C::ROWS_PER_Q) == 0, "a wave's rows never straddle K and V^T");
      if (C::ROWS_PER_Q * wu * C::QW < 64) {
        const uint8_t* base = k_base + (size_t)t * AKT * k_row_bytes;
#pragma unroll
        for (int j = 0; j < C::QW; ++j) dma16(base + src_off[j], stage + (wu * C::QW + j) * 1024);
      } else {
        const uint8_t* base = v_base + (size_t)t * AKT * C::ES;
#pragma unroll
        for (int j = 0; j < C::QW; ++j) dma16(base + src_off[j], stage + (wu * C::QW + j) * 1024);
      }
    } else {
#pragma unroll
      for (int j = 0; j < C::QW; ++j) {
        const int q = wu * C::QW + j;
        const int row = C::ROWS_PER_Q * q + lrow;
        const size_t chunk = (size_t)((lslot ^ (row & 7)) * 16);
        const uint8_t* src;
        if (C::ROWS_PER_Q * q < 64) {
          const int kr = min(j_first + t * AKT + row, T - 1);
          src = k_base + (size_t)kr * k_row_bytes + chunk;
        } else {
          src = v_base + ((size_t)(row - 64) * vt_stride + (size_t)t * AKT) * C::ES + chunk;
        }
        dma16(src, stage + q * 1024);
      }
    }
  };

  f32x4 oacc[NQ][4];
  float m_run[NQ], l_run[NQ];
  // bf16: the running sum of P comes from the matrix cores (an all-ones
  // block of V^T rows), every register of lacc holding the lane's query sum
  f32x4 lacc[NQ];
#pragma unroll
  for (int qt = 0; qt < NQ; ++qt) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[qt] = NEG_INF;
    l_run[qt] = 0.f;
    lacc[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // 8 in log2 units, as a difference of raw scores: P stays <= 256 (no
  // overflow in fp32 or bf16; bf16 rounds P to the same relative precision)
  const float lazy_gap = 8.f / scale_log2;
  for (int t = 0; t < C::STAGES - 1 && t < n_tiles; ++t) issue(t);
  for (int t = 0; t < n_tiles; ++t) {
    // this wave's loads of tile t (and the Q loads before them) are done
    // once at most `ahead` younger tiles of its loads remain in flight; the
    // barrier publishes every wave's and frees the stage of tile t - 1
    wait_vm(min(n_tiles - 1 - t, C::STAGES - 2) * C::QW);
    __builtin_amdgcn_s_barrier();
    if (t + C::STAGES - 1 < n_tiles) issue(t + C::STAGES - 1);
    const int j0 = j_first + t * AKT;
    if (!wave_any || j0 >= wk_hi || j0 + AKT <= wk_lo) continue;
    const uint8_t* Ks = smem + (t % C::STAGES) * C::TILE;
    const uint8_t* Vs = Ks + 64 * C::ROWB;

    // ---- S^T = K Q^T: lane holds keys 16 mt + 4 g + r of query li of
    // each query tile; a K fragment serves all NQ query tiles ----
    f32x4 sacc[NQ][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int qt = 0; qt < NQ; ++qt) sacc[qt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint8_t* kr = Ks + (16 * mt + li) * C::ROWB;
      if constexpr (PREC == P_F32) {
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(kr + (((4 * kc + g) ^ (li & 7)) << 4));
#pragma unroll
          for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int qt = 0; qt < NQ; ++qt)
              sacc[qt][mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], qf[qt][kc][s], sacc[qt][mt], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(kr + (((4 * kc + g) ^ (li & 7)) << 4));
#pragma unroll
          for (int qt = 0; qt < NQ; ++qt)
            sacc[qt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[qt][kc], sacc[qt][mt], 0, 0, 0);
        }
      }
    }

    // ---- mask, online softmax, per query tile.  The lane holds keys
    // j0 + 16 mt + 4 g + r of its query; key kj is allowed iff
    // kj - k_lo < k_span (unsigned).  A tile whose keys every lane of the
    // wave may all see skips the test ----
    float sv[NQ][16];
#pragma unroll
    for (int qt = 0; qt < NQ; ++qt) {
      const int kb = j0 + 4 * g - k_lo[qt];  // key offset of element (0, 0) from k_lo
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) sv[qt][mt * 4 + r] = sacc[qt][mt][r];
      if (!__all((unsigned)kb < k_span[qt] && (unsigned)(kb + 51) < k_span[qt])) {
        // some key of the tile is outside some lane's range: mask in place
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (!((unsigned)(kb + 16 * mt + r) < k_span[qt])) sv[qt][mt * 4 + r] = NEG_INF;
      }
      float mloc = NEG_INF;
#pragma unroll
      for (int i = 0; i < 16; ++i) mloc = fmaxf(mloc, sv[qt][i]);
      mloc = rows_max(mloc);
      // the reference max m_run moves to the running max only when that
      // exceeds it by more than lazy_gap (never while every score seen is
      // masked); the output and sum are then rescaled by exp2 of a
      // difference <= 0 (or -inf, giving 0), on the lanes that move
      const float m_new = fmaxf(m_run[qt], mloc);
      const bool move = m_new > m_run[qt] + lazy_gap;
      if (__any(move)) {
        const float m_use = m_new == NEG_INF ? 0.f : m_new;
        const float alpha = move ? __builtin_amdgcn_exp2f((m_run[qt] - m_use) * scale_log2) : 1.f;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) oacc[qt][dt] *= alpha;
        if constexpr (PREC == P_F32) l_run[qt] *= alpha;
        else lacc[qt] *= alpha;
        m_run[qt] = move ? m_new : m_run[qt];
      }
      // exponents <= 8 (scores at most lazy_gap above the reference)
      const float mb = (m_run[qt] == NEG_INF ? 0.f : m_run[qt]) * scale_log2;
#pragma unroll
      for (int i = 0; i < 16; ++i) sv[qt][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[qt][i], scale_log2, -mb));
      if constexpr (PREC == P_F32) {
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) psum += sv[qt][i];
        l_run[qt] += rows_sum(psum);
      }
    }

    // ---- O^T += V^T P^T; a V^T fragment serves all NQ query tiles ----
    if constexpr (PREC == P_F32) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const uint8_t* vr = Vs + (16 * dt + li) * C::ROWB;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(vr + (((4 * mt + g) ^ (li & 7)) << 4));
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int qt = 0; qt < NQ; ++qt)
              oacc[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r], sv[qt][mt * 4 + r], oacc[qt][dt], 0, 0, 0);
        }
      }
    } else {
      // P to bf16 with the pack-convert instruction (round to nearest even,
      // as f32_to_bf16 for the finite values here)
      bf16x8 pb[NQ][2];
      const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
#pragma unroll
      for (int qt = 0; qt < NQ; ++qt) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const u32x4 tt = {pack_bf16x2(sv[qt][8 * u + 0], sv[qt][8 * u + 1]),
                            pack_bf16x2(sv[qt][8 * u + 2], sv[qt][8 * u + 3]),
                            pack_bf16x2(sv[qt][8 * u + 4], sv[qt][8 * u + 5]),
                            pack_bf16x2(sv[qt][8 * u + 6], sv[qt][8 * u + 7])};
          pb[qt][u] = __builtin_bit_cast(bf16x8, tt);
          // sum of the (bf16) P of each query: ones x P^T
          lacc[qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[qt][u], lacc[qt], 0, 0, 0);
        }
      }
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const uint8_t* vr = Vs + (16 * dt + li) * C::ROWB;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          // keys 32u + 4g .. +3 and 32u + 16 + 4g .. +3 (the key order of
          // pb): columns 32u + 8g .. +7 of the tile in the bf16 V^T order
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(vr + (((4 * u + g) ^ (li & 7)) << 4));
#pragma unroll
          for (int qt = 0; qt < NQ; ++qt)
            oacc[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[qt][u], oacc[qt][dt], 0, 0, 0);
        }
      }
    }
  }

  // lane holds dims 16 dt + 4 g + r of query qi of each query tile
#pragma unroll
  for (int qt = 0; qt < NQ; ++qt) {
    if (qi[qt] >= q_end) continue;
    const float inv_l = 1.f / (PREC == P_BF16 ? lacc[qt][0] : l_run[qt]);
    if constexpr (PREC == P_F32) {
      float* op = reinterpret_cast<float*>(out) + (size_t)qi[qt] * H + h * 64;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) *reinterpret_cast<f32x4*>(op + 16 * dt + 4 * g) = oacc[qt][dt] * inv_l;
    } else {
      uint16_t* op = reinterpret_cast<uint16_t*>(out) + (size_t)qi[qt] * H + h * 64;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const uint32_t lo = pack_bf16x2(oacc[qt][dt][0] * inv_l, oacc[qt][dt][1] * inv_l);
        const uint32_t hi = pack_bf16x2(oacc[qt][dt][2] * inv_l, oacc[qt][dt][3] * inv_l);
        *reinterpret_cast<uint2*>(op + 16 * dt + 4 * g) = make_uint2(lo, hi);
      }
    }
  }
}

// RoPE of Q and K and transposition of V from an unrotated qkv (the same
// arithmetic as the QKV projection's epilogue): one thread per token and
// (head, pair) index c < H/2.
template <int PREC>
__global__ __launch_bounds__(256) void k_qkv_prep(const void* __restrict__ in, void* __restrict__ qk_out, QkvOut qo,
                                                  int T) {
  const int H = qo.hidden, half = H / 2;
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)T * half) return;
  const int t = (int)(idx / half), c = (int)(idx % half);
  const int h = c / 32, d = c % 32;
  const int pos = t - qo.seg[t].start;
  const float cs = qo.cos_tab[pos * 32 + d], sn = qo.sin_tab[pos * 32 + d];
  const size_t row = (size_t)t * 3 * H;
  auto ld = [&](size_t i) -> float {
    if constexpr (PREC == P_F32) return reinterpret_cast<const float*>(in)[i];
    else return bf16_to_f32(reinterpret_cast<const uint16_t*>(in)[i]);
  };
  auto st = [&](void* base, size_t i, float v) {
    if constexpr (PREC == P_F32) reinterpret_cast<float*>(base)[i] = v;
    else reinterpret_cast<uint16_t*>(base)[i] = f32_to_bf16(v);
  };
#pragma unroll
  for (int part = 0; part < 2; ++part) {  // Q, then K
    const size_t a = row + part * H + h * 64 + d;
    const float x = ld(a), y = ld(a + 32);
    st(qk_out, a, x * cs - y * sn);
    st(qk_out, a + 32, y * cs + x * sn);
  }
  const size_t v = row + 2 * H + h * 64 + d;
  const int col = PREC == P_BF16 ? vt_col_bf16(t) : t;
  st(qo.vt, (size_t)(h * 64 + d) * qo.vt_stride + col, ld(v));
  st(qo.vt, (size_t)(h * 64 + d + 32) * qo.vt_stride + col, ld(v + 32));
}

}  // namespace

void launch_attention(int prec, const void* qk, const void* vt, int vt_stride, void* o, const Seg* seg, int T,
                      int n_heads, int is_global, int window, int mean_len, hipStream_t s, const int* d_off,
                      const int* d_qunit, int n_texts) {
  if (T <= 0) return;
  const float scale_log2 = 0.125f * 1.4426950408889634f;
  // a double buffer: deeper rings (3 or 4 stages) measured slower on MI355X
  constexpr int ST = 2;
  // dynamic LDS above 64 KB must be allowed once (call_once: several host
  // threads may launch at the same time)
  static std::once_flag attr_once;
  std::call_once(attr_once, [] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn<P_BF16, ST, 1>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, AttnCfg<P_BF16, ST>::LDS);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn<P_BF16, ST, 2>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, AttnCfg<P_BF16, ST>::LDS);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn<P_F32, ST, 1>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, AttnCfg<P_F32, ST>::LDS);
  });
  if (prec == P_BF16) {
    // global layers over long texts: 32 queries per wave (128 per block),
    // each K / V^T fragment feeding two query tiles (4 texts of 4096: 3.4 ->
    // 3.0 ms of global attention per pass).  Short texts and local layers
    // keep 16: a 128-query block spans more texts' keys (packs of texts of
    // ~190 tokens: 11.5 -> 8.8 ms per 64-pack step with 64-query blocks;
    // local layers over 4096-token texts: 0.58 -> 0.70 ms with 128).
    if (is_global && mean_len >= 1024) {
      const dim3 grid((T + 127) / 128, n_heads);
      launch_timed(k_attn<P_BF16, ST, 2>, grid, dim3(256), AttnCfg<P_BF16, ST>::LDS, s, qk, vt, vt_stride, o, seg, T,
                   n_heads, is_global, window, scale_log2, (const int*)nullptr, (const int*)nullptr, 0);
      return;
    }
  }
  // 64-query blocks.  On global layers with the per-text units (d_qunit)
  // a block never spans two texts, so it walks one text's keys instead of
  // the union of several (packs of texts of ~120 tokens: 8.4 -> 7.7 ms of
  // global attention per 64-pack step); the grid covers sum over texts of
  // ceil(len / 64) <= (T + 63 B) / 64 units.  Local layers keep blocks of
  // consecutive queries: a window reaches at most 64 tokens either way, and
  // text-aligned blocks there only add part-empty blocks (7.5 -> 9.8 ms).
  if (!is_global) d_qunit = nullptr;
  const dim3 grid(d_qunit ? (T + (ATTN_QUNIT - 1) * n_texts) / ATTN_QUNIT : (T + 63) / 64, n_heads);
  if (prec == P_BF16)
    launch_timed(k_attn<P_BF16, ST, 1>, grid, dim3(256), AttnCfg<P_BF16, ST>::LDS, s, qk, vt, vt_stride, o, seg, T,
                 n_heads, is_global, window, scale_log2, d_off, d_qunit, n_texts);
  else
    launch_timed(k_attn<P_F32, ST, 1>, grid, dim3(256), AttnCfg<P_F32, ST>::LDS, s, qk, vt, vt_stride, o, seg, T,
                 n_heads, is_global, window, scale_log2, d_off, d_qunit, n_texts);
}

void launch_qkv_prep(int prec, const void* qkv_in, void* qk_out, const QkvOut& qo, int T, hipStream_t s) {
  if (T <= 0) return;
  const long n = (long)T * (qo.hidden / 2);
  const int blocks = (int)((n + 255) / 256);
  if (prec == P_BF16) k_qkv_prep<P_BF16><<<blocks, 256, 0, s>>>(qkv_in, qk_out, qo, T);
  else k_qkv_prep<P_F32><<<blocks, 256, 0, s>>>(qkv_in, qk_out, qo, T);
}

}  // namespace tte
