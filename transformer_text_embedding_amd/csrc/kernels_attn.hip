// Attention over a pack of texts, one head per block column, with RoPE
// applied to Q and K as they are loaded.
//
// What it computes (tensai "テキスト埋め込み" page, section 何が動くか):
// every token attends to the tokens of its own text in both directions; on
// a global layer to all of them, on a local layer only to those at most
// `window` positions away; RoPE positions restart at 0 in every text
// (packing paragraph), base 160000 on global layers and 10000 on local ones
// (encoder paragraph).  Score = q.k / sqrt(64), softmax over the allowed
// keys, output = sum of p * v.
//
// How: flash-style streaming over the packed token axis.  A block takes 64
// consecutive queries (they may span several texts) and walks 64-key tiles
// over the union of their allowed key ranges only: for a local layer that
// is at most 64 + 2*window keys, for a global one the texts the queries
// belong to, so fully masked tiles are never visited; a wave additionally
// skips the matrix work of tiles outside its own 16 queries' window.  Inside
// a tile the mask is (same text) and (global or |i - j| <= window), taken per
// element from the per-token text bounds.
//
// The products are taken transposed, S^T = K Q^T and O^T = V^T P^T, so that
// the matrix-core output layout puts one query per lane column: each lane's
// scores of its query are then directly the B operand of the P*V product,
// and the running max / sum / rescale of a query live in the lanes that hold
// it, with two cross-lane steps per reduction.  Softmax uses exp2 with
// log2(e)/8 folded into one multiply.  fp32 variant: v_mfma_f32_16x16x4_f32;
// bf16 variant: v_mfma_f32_16x16x32_bf16 with Q, K (after RoPE), V and P
// rounded to bf16 and all statistics in fp32.
#include "common.h"
#include "kernels.h"

namespace tte {

namespace {

constexpr int AQ = 64;  // queries per block
constexpr int AKT = 64; // keys per tile
constexpr float NEG_INF = -__builtin_huge_valf();

template <int PREC>
struct AttnLds;

template <>
struct AttnLds<P_F32> {
  float k[AKT][68];   // K tile after RoPE, [key][dim]
  float vt[64][68];   // V tile transposed, [dim][key]
  int kseg[AKT];      // text start of each key (-2: outside the range)
};

template <>
struct AttnLds<P_BF16> {
  uint16_t k[AKT][72];
  uint16_t vt[64][72];
  int kseg[AKT];
};

template <int PREC>
__global__ __launch_bounds__(256) void k_attn(const void* __restrict__ qkv, void* __restrict__ out,
                                              const Seg* __restrict__ seg, const float* __restrict__ cos_tab,
                                              const float* __restrict__ sin_tab, int T, int nh, int is_global,
                                              int window, float scale_log2) {
  __shared__ AttnLds<PREC> sm;
  const int H = nh * 64, ld = 3 * H;
  const int h = blockIdx.y;
  const int i0 = blockIdx.x * AQ;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, li = lane & 15;

  const int ilast = min(i0 + AQ - 1, T - 1);
  const Seg sa = seg[i0], sb = seg[ilast];
  int kstart = sa.start, kend = sb.end;
  if (!is_global) {
    kstart = max(kstart, i0 - window);
    kend = min(kend, ilast + window + 1);
  }
  const int wq_lo = i0 + 16 * w, wq_hi = min(i0 + 16 * w + 15, T - 1);

  const int qi = i0 + 16 * w + li;
  const bool qvalid = qi < T;
  const int qrow = qvalid ? qi : T - 1;
  const Seg qs = seg[qrow];
  const int qseg = qvalid ? qs.start : -1;
  const int qpos = qrow - qs.start;

  // ---- Q fragment with RoPE (pairs (d, d+32)) ----
  f32x4 qf[4];      // fp32: dims 16 kc + 4 g + e
  bf16x8 qb[2];     // bf16: dims 32 kc + 8 g + e
  if constexpr (PREC == P_F32) {
    const float* qp = reinterpret_cast<const float*>(qkv) + (size_t)qrow * ld + h * 64;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) qf[kc] = *reinterpret_cast<const f32x4*>(qp + 16 * kc + 4 * g);
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const f32x4 c = *reinterpret_cast<const f32x4*>(cos_tab + qpos * 32 + 16 * kc + 4 * g);
      const f32x4 s = *reinterpret_cast<const f32x4*>(sin_tab + qpos * 32 + 16 * kc + 4 * g);
      const f32x4 x = qf[kc], y = qf[kc + 2];
      qf[kc] = x * c - y * s;
      qf[kc + 2] = y * c + x * s;
    }
  } else {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(qkv) + (size_t)qrow * ld + h * 64;
    const u16x8 r0 = *reinterpret_cast<const u16x8*>(qp + 8 * g);
    const u16x8 r1 = *reinterpret_cast<const u16x8*>(qp + 32 + 8 * g);
    u16x8 o0, o1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float c = cos_tab[qpos * 32 + 8 * g + e], s = sin_tab[qpos * 32 + 8 * g + e];
      const float x = bf16_to_f32(r0[e]), y = bf16_to_f32(r1[e]);
      o0[e] = f32_to_bf16(x * c - y * s);
      o1[e] = f32_to_bf16(y * c + x * s);
    }
    qb[0] = __builtin_bit_cast(bf16x8, o0);
    qb[1] = __builtin_bit_cast(bf16x8, o1);
  }

  f32x4 oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = NEG_INF, l_run = 0.f;

  for (int j0 = kstart; j0 < kend; j0 += AKT) {
    __syncthreads();
    // ---- K tile (RoPE) and transposed V tile into LDS ----
    if constexpr (PREC == P_F32) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int p = tid + 256 * i, key = p >> 3, c = p & 7;
        const int kj = j0 + key, krow = min(kj, T - 1);
        const Seg ks = seg[krow];
        const int kpos = krow - ks.start;
        const float* kp = reinterpret_cast<const float*>(qkv) + (size_t)krow * ld + H + h * 64;
        const f32x4 x = *reinterpret_cast<const f32x4*>(kp + 4 * c);
        const f32x4 y = *reinterpret_cast<const f32x4*>(kp + 32 + 4 * c);
        const f32x4 cs = *reinterpret_cast<const f32x4*>(cos_tab + kpos * 32 + 4 * c);
        const f32x4 sn = *reinterpret_cast<const f32x4*>(sin_tab + kpos * 32 + 4 * c);
        *reinterpret_cast<f32x4*>(&sm.k[key][4 * c]) = x * cs - y * sn;
        *reinterpret_cast<f32x4*>(&sm.k[key][32 + 4 * c]) = y * cs + x * sn;
        if (c == 0) sm.kseg[key] = kj < kend ? ks.start : -2;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = tid + 256 * i, key = p >> 4, c4 = p & 15;
        const int krow = min(j0 + key, T - 1);
        const f32x4 v =
            *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(qkv) + (size_t)krow * ld + 2 * H + h * 64 + 4 * c4);
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.vt[4 * c4 + e][key] = v[e];
      }
    } else {
      {
        const int key = tid >> 2, c = tid & 3;
        const int kj = j0 + key, krow = min(kj, T - 1);
        const Seg ks = seg[krow];
        const int kpos = krow - ks.start;
        const uint16_t* kp = reinterpret_cast<const uint16_t*>(qkv) + (size_t)krow * ld + H + h * 64;
        const u16x8 x = *reinterpret_cast<const u16x8*>(kp + 8 * c);
        const u16x8 y = *reinterpret_cast<const u16x8*>(kp + 32 + 8 * c);
        u16x8 o0, o1;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float cs = cos_tab[kpos * 32 + 8 * c + e], sn = sin_tab[kpos * 32 + 8 * c + e];
          const float xf = bf16_to_f32(x[e]), yf = bf16_to_f32(y[e]);
          o0[e] = f32_to_bf16(xf * cs - yf * sn);
          o1[e] = f32_to_bf16(yf * cs + xf * sn);
        }
        *reinterpret_cast<u16x8*>(&sm.k[key][8 * c]) = o0;
        *reinterpret_cast<u16x8*>(&sm.k[key][32 + 8 * c]) = o1;
        if (c == 0) sm.kseg[key] = kj < kend ? ks.start : -2;
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int p = tid + 256 * i, key = p >> 3, c8 = p & 7;
        const int krow = min(j0 + key, T - 1);
        const u16x8 v = *reinterpret_cast<const u16x8*>(reinterpret_cast<const uint16_t*>(qkv) + (size_t)krow * ld +
                                                        2 * H + h * 64 + 8 * c8);
#pragma unroll
        for (int e = 0; e < 8; ++e) sm.vt[8 * c8 + e][key] = v[e];
      }
    }
    __syncthreads();

    if (!is_global && (j0 > wq_hi + window || j0 + AKT - 1 < wq_lo - window)) continue;

    // ---- S^T = K Q^T: lane holds keys 16 mt + 4 g + r of query li ----
    f32x4 sacc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      sacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (PREC == P_F32) {
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(&sm.k[16 * mt + li][16 * kc + 4 * g]);
#pragma unroll
          for (int s = 0; s < 4; ++s) sacc[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], qf[kc][s], sacc[mt], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sm.k[16 * mt + li][32 * kc + 8 * g]);
          sacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[kc], sacc[mt], 0, 0, 0);
        }
      }
    }

    // ---- mask, online softmax ----
    float sv[16];
    float mloc = NEG_INF;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kk = 16 * mt + 4 * g + r;
        const int kj = j0 + kk;
        const int d = qi - kj;
        const bool ok = (sm.kseg[kk] == qseg) && (is_global || (d <= window && -d <= window));
        sv[mt * 4 + r] = ok ? sacc[mt][r] : NEG_INF;
        mloc = fmaxf(mloc, sv[mt * 4 + r]);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    const float m_new = fmaxf(m_run, mloc);
    const float m_use = m_new == NEG_INF ? 0.f : m_new;
    const float alpha = exp2f((m_run - m_use) * scale_log2);
    const float mb = m_use * scale_log2;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sv[i] = exp2f(__builtin_fmaf(sv[i], scale_log2, -mb));
      psum += sv[i];
    }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[dt] *= alpha;

    // ---- O^T += V^T P^T ----
    if constexpr (PREC == P_F32) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(&sm.vt[16 * dt + li][16 * mt + 4 * g]);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r], sv[mt * 4 + r], oacc[dt], 0, 0, 0);
        }
    } else {
      bf16x8 pb[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        u16x8 t;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          t[e] = f32_to_bf16(sv[(2 * u) * 4 + e]);
          t[4 + e] = f32_to_bf16(sv[(2 * u + 1) * 4 + e]);
        }
        pb[u] = __builtin_bit_cast(bf16x8, t);
      }
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const u16x4 lo = *reinterpret_cast<const u16x4*>(&sm.vt[16 * dt + li][32 * u + 4 * g]);
          const u16x4 hi = *reinterpret_cast<const u16x4*>(&sm.vt[16 * dt + li][32 * u + 16 + 4 * g]);
          const u16x8 t = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, t), pb[u], oacc[dt], 0, 0, 0);
        }
    }
  }

  if (!qvalid) return;
  const float inv_l = 1.f / l_run;
  // lane holds dims 16 dt + 4 g + r of query qi
  if constexpr (PREC == P_F32) {
    float* op = reinterpret_cast<float*>(out) + (size_t)qi * H + h * 64;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) *reinterpret_cast<f32x4*>(op + 16 * dt + 4 * g) = oacc[dt] * inv_l;
  } else {
    uint16_t* op = reinterpret_cast<uint16_t*>(out) + (size_t)qi * H + h * 64;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const u16x4 t = {f32_to_bf16(oacc[dt][0] * inv_l), f32_to_bf16(oacc[dt][1] * inv_l),
                       f32_to_bf16(oacc[dt][2] * inv_l), f32_to_bf16(oacc[dt][3] * inv_l)};
      *reinterpret_cast<u16x4*>(op + 16 * dt + 4 * g) = t;
    }
  }
}

}  // namespace

void launch_attention(int prec, const void* qkv, void* o, const Seg* seg, const float* cos_tab, const float* sin_tab,
                      int T, int n_heads, int is_global, int window, hipStream_t s) {
  if (T <= 0) return;
  const dim3 grid((T + AQ - 1) / AQ, n_heads);
  const float scale_log2 = 0.125f * 1.4426950408889634f;
  if (prec == P_BF16)
    k_attn<P_BF16><<<grid, 256, 0, s>>>(qkv, o, seg, cos_tab, sin_tab, T, n_heads, is_global, window, scale_log2);
  else
    k_attn<P_F32><<<grid, 256, 0, s>>>(qkv, o, seg, cos_tab, sin_tab, T, n_heads, is_global, window, scale_log2);
}

}  // namespace tte
