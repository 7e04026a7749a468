// NT GEMM on the gfx950 matrix cores: C[M, N] = A[M, K] * W[N, K]^T, both
// operands contiguous along K.  These are the encoder's four weight products
// (QKV, attention output, GeGLU up-projection, down-projection) of the tensai
// "テキスト埋め込み" page, section 何が動くか (encoder paragraph); the int8
// form is the integer matmul of its section 精度と量子化.
//
// One kernel template serves three operand formats.  Every K tile is 128
// bytes per row whatever the format (32 fp32, 64 bf16 or 128 int8), so the
// global->LDS traffic is identical: a 128 x 128 output tile, 256 threads
// (4 waves in a 2 x 2 grid, each owning 64 x 64 = 4 x 4 MFMA 16x16 tiles),
// A and W tiles of 128 rows x 128 bytes double-buffered in LDS with rows
// padded to 144 bytes (16-lane fragment reads land in distinct banks), the
// next K tile prefetched into registers while the current one is consumed.
//
//   fp32: v_mfma_f32_16x16x4_f32, 4 per 16-k chunk (each lane reads a float4
//         and feeds one element per MFMA; A and W use the same k order).
//   bf16: v_mfma_f32_16x16x32_bf16, one per 32-k chunk, fp32 accumulate.
//   int8: v_mfma_i32_16x16x32_i8, one per 32-k block (exact int32 sum of the
//         block), then acc += float(sum) * w_scale[n, block] in fp32; the row
//         scale a_scale[m] multiplies once in the epilogue.
//
// Epilogues: STORE (fp32 or bf16), RESID (fp32 C += result), GEGLU.  For
// GEGLU the W tile rows are chosen so that every wave's first 32 columns
// are up-projection rows n (the GELU half) and its last 32 are rows I + n
// (the gate half): the two halves of one output land in the same lane and
// combine in registers, and the [M, 2I] intermediate is never stored.
#include "common.h"
#include "kernels.h"

namespace tte {

namespace {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int KT_BYTES = 128;  // bytes of K per tile row
constexpr int LDS_ROW = 144;   // padded LDS row (bytes)
constexpr int STAGE = (BM + BN) * LDS_ROW;

template <int PREC>
struct Fmt {
  static constexpr int ES = PREC == P_F32 ? 4 : (PREC == P_BF16 ? 2 : 1);
  static constexpr int BK = KT_BYTES / ES;
};

// Row of W that tile row r (0..127) of n-block nb reads.
template <int EPI>
__device__ __forceinline__ int w_row(int r, int nb, int N) {
  if constexpr (EPI == E_GEGLU) {
    const int half_wave = r >> 6, within = r & 63;
    const int base = nb * 64 + half_wave * 32;
    return within < 32 ? base + within : N + base + (within - 32);
  } else {
    return nb * BN + r;
  }
}

// Global -> registers: one 16-byte chunk of 4 A rows and 4 W rows (and, for
// int8, the lane's 4 weight-scale vectors) of K tile kt.
template <int PREC>
__device__ __forceinline__ void fetch_tile(u32x4 (&ra)[4], u32x4 (&rw)[4], f32x4 (&sw)[4], const uint8_t* a_src0,
                                           const uint8_t* w_src0, const size_t (&a_off)[4], const size_t (&w_off)[4],
                                           const float* w_scale, const size_t (&s_off)[4], int kt) {
  const size_t k_off = (size_t)kt * KT_BYTES;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ra[i] = *reinterpret_cast<const u32x4*>(a_src0 + a_off[i] + k_off);
    rw[i] = *reinterpret_cast<const u32x4*>(w_src0 + w_off[i] + k_off);
  }
  if constexpr (PREC == P_I8) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) sw[nt] = *reinterpret_cast<const f32x4*>(w_scale + s_off[nt] + kt * 4);
  }
}

__device__ __forceinline__ void stash_tile(uint8_t* base, const u32x4 (&ra)[4], const u32x4 (&rw)[4], int lrow,
                                           int lch) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    *reinterpret_cast<u32x4*>(base + (lrow + 32 * i) * LDS_ROW + lch * 16) = ra[i];
    *reinterpret_cast<u32x4*>(base + (BM + lrow + 32 * i) * LDS_ROW + lch * 16) = rw[i];
  }
}

template <int PREC, int EPI, int OUT>
__global__ __launch_bounds__(256) void k_gemm(const uint8_t* __restrict__ A, const float* __restrict__ a_scale,
                                              const uint8_t* __restrict__ W, const float* __restrict__ w_scale,
                                              void* __restrict__ C, int M, int N, int K) {
  using F = Fmt<PREC>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int g = lane >> 4, li = lane & 15;
  const int nb = blockIdx.x, m0 = blockIdx.y * BM;
  const size_t row_bytes = (size_t)K * F::ES;
  const int nk = K / F::BK;

  // global -> register assignment: rows lrow + 32 i, 16-byte chunk lch
  const int lrow = tid >> 3, lch = tid & 7;
  const uint8_t* a_src0 = A + lch * 16;
  const uint8_t* w_src0 = W + lch * 16;
  size_t a_off[4], w_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a_off[i] = (size_t)min(m0 + lrow + 32 * i, M - 1) * row_bytes;
    w_off[i] = (size_t)w_row<EPI>(lrow + 32 * i, nb, N) * row_bytes;
  }

  // int8: per-lane weight scales of its 4 column groups, 4 blocks per K tile
  const int kblocks = K / 32;
  size_t s_off[4] = {0, 0, 0, 0};
  if constexpr (PREC == P_I8) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) s_off[nt] = (size_t)w_row<EPI>(wn * 64 + nt * 16 + li, nb, N) * kblocks;
  }

  u32x4 ra[4], rw[4];
  f32x4 sw[4], sw_next[4];

  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  fetch_tile<PREC>(ra, rw, sw_next, a_src0, w_src0, a_off, w_off, w_scale, s_off, 0);
  stash_tile(smem, ra, rw, lrow, lch);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if constexpr (PREC == P_I8) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) sw[nt] = sw_next[nt];
    }
    if (kt + 1 < nk) fetch_tile<PREC>(ra, rw, sw_next, a_src0, w_src0, a_off, w_off, w_scale, s_off, kt + 1);
    const uint8_t* As = smem + cur * STAGE + (wm * 64 + li) * LDS_ROW;
    const uint8_t* Bs = smem + cur * STAGE + (BM + wn * 64 + li) * LDS_ROW;

    if constexpr (PREC == P_F32) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        f32x4 af[4], bf[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          af[t] = *reinterpret_cast<const f32x4*>(As + t * 16 * LDS_ROW + c * 64 + g * 16);
          bf[t] = *reinterpret_cast<const f32x4*>(Bs + t * 16 * LDS_ROW + c * 64 + g * 16);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
              acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[mt][s], bf[nt][s], acc[mt][nt], 0, 0, 0);
      }
    } else if constexpr (PREC == P_BF16) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        bf16x8 af[4], bf[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          af[t] = *reinterpret_cast<const bf16x8*>(As + t * 16 * LDS_ROW + c * 64 + g * 16);
          bf[t] = *reinterpret_cast<const bf16x8*>(Bs + t * 16 * LDS_ROW + c * 64 + g * 16);
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mt], bf[nt], acc[mt][nt], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        long af[4], bf[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          af[t] = *reinterpret_cast<const long*>(As + t * 16 * LDS_ROW + c * 32 + g * 8);
          bf[t] = *reinterpret_cast<const long*>(Bs + t * 16 * LDS_ROW + c * 32 + g * 8);
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) {
            const i32x4 p = __builtin_amdgcn_mfma_i32_16x16x32_i8(af[mt], bf[nt], i32x4{0, 0, 0, 0}, 0, 0, 0);
            const float s = sw[nt][c];
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[mt][nt][r] = __builtin_fmaf((float)p[r], s, acc[mt][nt][r]);
          }
      }
    }

    if (kt + 1 < nk) stash_tile(smem + (cur ^ 1) * STAGE, ra, rw, lrow, lch);
    __syncthreads();
  }

  // epilogue: lane holds rows 4g + r of column li in every 16 x 16 tile
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + wm * 64 + mt * 16 + 4 * g + r;
      if (m >= M) continue;
      float rs = 1.f;
      if constexpr (PREC == P_I8) rs = a_scale[m];
      if constexpr (EPI == E_GEGLU) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int n = nb * 64 + wn * 32 + nt * 16 + li;
          const float v = gelu_erf(acc[mt][nt][r] * rs) * (acc[mt][nt + 2][r] * rs);
          if constexpr (OUT == O_BF16) reinterpret_cast<uint16_t*>(C)[(size_t)m * N + n] = f32_to_bf16(v);
          else reinterpret_cast<float*>(C)[(size_t)m * N + n] = v;
        }
      } else {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const int n = nb * BN + wn * 64 + nt * 16 + li;
          const float v = acc[mt][nt][r] * rs;
          if constexpr (EPI == E_RESID) {
            reinterpret_cast<float*>(C)[(size_t)m * N + n] += v;
          } else if constexpr (OUT == O_BF16) {
            reinterpret_cast<uint16_t*>(C)[(size_t)m * N + n] = f32_to_bf16(v);
          } else {
            reinterpret_cast<float*>(C)[(size_t)m * N + n] = v;
          }
        }
      }
    }
  }
}

template <int PREC, int EPI, int OUT>
void go(const void* A, const float* a_scale, const void* W, const float* w_scale, int M, int N, int K, void* C,
        hipStream_t s) {
  const int nblocks = EPI == E_GEGLU ? N / 64 : N / BN;
  const dim3 grid(nblocks, (M + BM - 1) / BM);
  k_gemm<PREC, EPI, OUT><<<grid, 256, 0, s>>>(reinterpret_cast<const uint8_t*>(A), a_scale,
                                               reinterpret_cast<const uint8_t*>(W), w_scale, C, M, N, K);
}

template <int PREC>
void go_prec(int epi, const void* A, const float* a_scale, const void* W, const float* w_scale, int M, int N, int K,
             void* C, int out_kind, hipStream_t s) {
  if (epi == E_RESID) {
    go<PREC, E_RESID, O_F32>(A, a_scale, W, w_scale, M, N, K, C, s);
  } else if (epi == E_GEGLU) {
    if (out_kind == O_BF16) go<PREC, E_GEGLU, O_BF16>(A, a_scale, W, w_scale, M, N, K, C, s);
    else go<PREC, E_GEGLU, O_F32>(A, a_scale, W, w_scale, M, N, K, C, s);
  } else {
    if (out_kind == O_BF16) go<PREC, E_STORE, O_BF16>(A, a_scale, W, w_scale, M, N, K, C, s);
    else go<PREC, E_STORE, O_F32>(A, a_scale, W, w_scale, M, N, K, C, s);
  }
}

}  // namespace

void launch_gemm(int prec, int epi, const void* A, const float* a_scale, const void* W, const float* w_scale, int M,
                 int N, int K, void* C, int out_kind, hipStream_t s) {
  if (M <= 0) return;
  if (prec == P_F32) go_prec<P_F32>(epi, A, a_scale, W, w_scale, M, N, K, C, out_kind, s);
  else if (prec == P_BF16) go_prec<P_BF16>(epi, A, a_scale, W, w_scale, M, N, K, C, out_kind, s);
  else go_prec<P_I8>(epi, A, a_scale, W, w_scale, M, N, K, C, out_kind, s);
}

}  // namespace tte
