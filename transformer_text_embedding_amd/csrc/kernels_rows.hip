// Row-wise kernels: embedding gather + LayerNorm, LayerNorm (fp32 / bf16 /
// 7-bit int8 output), per-row 7-bit quantisation, final LayerNorm + mean
// pool + L2.  All are HBM-bound; one wave64 owns one row, holds it in
// registers (width/64 values per lane, loaded as 16-byte vectors where the
// width allows) and reduces with cross-lane shuffles, so each row is read
// once and written once.
//
// Bias-free LayerNorm, mean pooling and unit length follow the tensai
// "テキスト埋め込み" page, section 何が動くか (encoder and pooling
// paragraphs); the 7-bit row code follows its section 精度と量子化.
#include "common.h"
#include "kernels.h"

namespace tte {

template <int EPL>
struct RowShape {
  static constexpr int VEC = (EPL % 4 == 0) ? 4 : ((EPL % 2 == 0) ? 2 : 1);
  static constexpr int CH = EPL / VEC;
  static constexpr int W = EPL * 64;
  __device__ static __forceinline__ int col(int c, int lane, int v) { return c * 64 * VEC + lane * VEC + v; }
};

template <int EPL>
__device__ __forceinline__ void load_f32_row(const float* __restrict__ row, int lane, float (&v)[EPL]) {
  using RS = RowShape<EPL>;
#pragma unroll
  for (int c = 0; c < RS::CH; ++c) {
    const float* p = row + RS::col(c, lane, 0);
    if constexpr (RS::VEC == 4) {
      float4 t = *reinterpret_cast<const float4*>(p);
      v[c * 4 + 0] = t.x; v[c * 4 + 1] = t.y; v[c * 4 + 2] = t.z; v[c * 4 + 3] = t.w;
    } else if constexpr (RS::VEC == 2) {
      float2 t = *reinterpret_cast<const float2*>(p);
      v[c * 2 + 0] = t.x; v[c * 2 + 1] = t.y;
    } else {
      v[c] = p[0];
    }
  }
}

template <int EPL>
__device__ __forceinline__ void store_f32_row(float* __restrict__ row, int lane, const float (&v)[EPL]) {
  using RS = RowShape<EPL>;
#pragma unroll
  for (int c = 0; c < RS::CH; ++c) {
    float* p = row + RS::col(c, lane, 0);
    if constexpr (RS::VEC == 4) {
      *reinterpret_cast<float4*>(p) = make_float4(v[c * 4 + 0], v[c * 4 + 1], v[c * 4 + 2], v[c * 4 + 3]);
    } else if constexpr (RS::VEC == 2) {
      *reinterpret_cast<float2*>(p) = make_float2(v[c * 2 + 0], v[c * 2 + 1]);
    } else {
      p[0] = v[c];
    }
  }
}

template <int EPL>
__device__ __forceinline__ void store_bf16_row(uint16_t* __restrict__ row, int lane, const float (&v)[EPL]) {
  using RS = RowShape<EPL>;
#pragma unroll
  for (int c = 0; c < RS::CH; ++c) {
    uint16_t* p = row + RS::col(c, lane, 0);
    if constexpr (RS::VEC == 4) {
      u16x4 t = {f32_to_bf16(v[c * 4 + 0]), f32_to_bf16(v[c * 4 + 1]), f32_to_bf16(v[c * 4 + 2]),
                 f32_to_bf16(v[c * 4 + 3])};
      *reinterpret_cast<u16x4*>(p) = t;
    } else {
#pragma unroll
      for (int e = 0; e < RS::VEC; ++e) p[e] = f32_to_bf16(v[c * RS::VEC + e]);
    }
  }
}

template <int EPL>
__device__ __forceinline__ void load_bf16_row(const uint16_t* __restrict__ row, int lane, float (&v)[EPL]) {
  using RS = RowShape<EPL>;
#pragma unroll
  for (int c = 0; c < RS::CH; ++c) {
    const uint16_t* p = row + RS::col(c, lane, 0);
    if constexpr (RS::VEC == 4) {
      const u16x4 t = *reinterpret_cast<const u16x4*>(p);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[c * 4 + e] = bf16_to_f32(t[e]);
    } else {
#pragma unroll
      for (int e = 0; e < RS::VEC; ++e) v[c * RS::VEC + e] = bf16_to_f32(p[e]);
    }
  }
}

// Row r of the residual stream x: fp32, or bf16 (XB) in the bf16 mode.
template <int EPL, bool XB>
__device__ __forceinline__ void load_x_row(const void* __restrict__ x, size_t r, int lane, float (&v)[EPL]) {
  if constexpr (XB) load_bf16_row<EPL>(reinterpret_cast<const uint16_t*>(x) + r * RowShape<EPL>::W, lane, v);
  else load_f32_row<EPL>(reinterpret_cast<const float*>(x) + r * RowShape<EPL>::W, lane, v);
}

// Stores row r of x; with XB the values are first rounded to bf16 in
// place, so that what the caller goes on to use is what x now holds.
template <int EPL, bool XB>
__device__ __forceinline__ void store_x_row(void* __restrict__ x, size_t r, int lane, float (&v)[EPL]) {
  if constexpr (XB) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) v[i] = bf16_to_f32(f32_to_bf16(v[i]));
    store_bf16_row<EPL>(reinterpret_cast<uint16_t*>(x) + r * RowShape<EPL>::W, lane, v);
  } else {
    store_f32_row<EPL>(reinterpret_cast<float*>(x) + r * RowShape<EPL>::W, lane, v);
  }
}

// 7-bit codes of a row held in registers; returns the row scale amax/63.
template <int EPL>
__device__ __forceinline__ float store_q7_row(int8_t* __restrict__ row, int lane, const float (&v)[EPL]) {
  using RS = RowShape<EPL>;
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = wave_max(amax);
  const float inv = amax > 0.f ? 63.f / amax : 0.f;
#pragma unroll
  for (int c = 0; c < RS::CH; ++c) {
    int8_t* p = row + RS::col(c, lane, 0);
    if constexpr (RS::VEC == 4) {
      uint32_t packed = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) packed |= ((uint32_t)(uint8_t)(int8_t)quant7(v[c * 4 + e], inv)) << (8 * e);
      *reinterpret_cast<uint32_t*>(p) = packed;
    } else {
#pragma unroll
      for (int e = 0; e < RS::VEC; ++e) p[e] = (int8_t)quant7(v[c * RS::VEC + e], inv);
    }
  }
  return amax > 0.f ? amax / 63.f : 0.f;
}

// In-register bias-free LayerNorm of one row: two passes over registers
// (mean, then centred sum of squares), fp32 statistics.
template <int EPL>
__device__ __forceinline__ void layernorm_regs(float (&v)[EPL], const float* __restrict__ gamma, int lane,
                                               float eps) {
  using RS = RowShape<EPL>;
  float g[EPL];
  load_f32_row<EPL>(gamma, lane, g);  // issued before the reductions
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) s += v[i];
  const float mean = wave_sum(s) * (1.f / RS::W);
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    v[i] -= mean;
    q += v[i] * v[i];
  }
  const float rstd = __builtin_amdgcn_rsqf(wave_sum(q) * (1.f / RS::W) + eps);
#pragma unroll
  for (int i = 0; i < EPL; ++i) v[i] = v[i] * rstd * g[i];
}

// --------------------------------------------------------------------------
// embedding gather + LayerNorm; per-token text bounds
// --------------------------------------------------------------------------

template <int EPL, int PREC, bool XB>
__global__ __launch_bounds__(256) void k_embed_ln(const int32_t* __restrict__ ids, const PackIO* __restrict__ io,
                                                  int T, const void* __restrict__ table,
                                                  const float* __restrict__ table_scale, int vocab,
                                                  const float* __restrict__ gamma, float eps,
                                                  const int* __restrict__ off, int n_texts,
                                                  void* __restrict__ x, Seg* __restrict__ seg) {
  using RS = RowShape<EPL>;
  constexpr int H = RS::W;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  if (io) ids = io->ids;
  int id = ids[t];
  id = id < 0 ? 0 : (id >= vocab ? vocab - 1 : id);
  const int b = wave_find(off, n_texts, t);  // the token's text (off strictly increasing, off[0] = 0)
  float v[EPL];
  if constexpr (PREC == P_F32) {
    load_f32_row<EPL>(reinterpret_cast<const float*>(table) + (size_t)id * H, lane, v);
  } else if constexpr (PREC == P_BF16) {
    const uint16_t* r = reinterpret_cast<const uint16_t*>(table) + (size_t)id * H;
#pragma unroll
    for (int c = 0; c < RS::CH; ++c)
#pragma unroll
      for (int e = 0; e < RS::VEC; ++e) v[c * RS::VEC + e] = bf16_to_f32(r[RS::col(c, lane, e)]);
  } else {
    const int8_t* r = reinterpret_cast<const int8_t*>(table) + (size_t)id * H;
    const float* sc = table_scale + (size_t)id * (H / 32);
#pragma unroll
    for (int c = 0; c < RS::CH; ++c)
#pragma unroll
      for (int e = 0; e < RS::VEC; ++e) {
        const int k = RS::col(c, lane, e);
        v[c * RS::VEC + e] = (float)r[k] * sc[k >> 5];
      }
  }
  layernorm_regs<EPL>(v, gamma, lane, eps);
  store_x_row<EPL, XB>(x, (size_t)t, lane, v);
  if (lane == 0) seg[t] = Seg{off[b], off[b + 1]};
}

// --------------------------------------------------------------------------
// LayerNorm / conversion / quantisation of fp32 (or, XB, bf16) rows
// --------------------------------------------------------------------------

template <int EPL, int OUT, bool NORM, bool XB>
__global__ __launch_bounds__(256) void k_ln(const void* __restrict__ x, const float* __restrict__ gamma, int rows,
                                            float eps, void* __restrict__ out, float* __restrict__ out_scale,
                                            const PackIO* __restrict__ io) {
  using RS = RowShape<EPL>;
  constexpr int Wd = RS::W;
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  if (io) out = io->out;
  float v[EPL];
  load_x_row<EPL, XB>(x, (size_t)r, lane, v);
  if constexpr (NORM) layernorm_regs<EPL>(v, gamma, lane, eps);
  if constexpr (OUT == O_F32) {
    store_f32_row<EPL>(reinterpret_cast<float*>(out) + (size_t)r * Wd, lane, v);
  } else if constexpr (OUT == O_BF16) {
    store_bf16_row<EPL>(reinterpret_cast<uint16_t*>(out) + (size_t)r * Wd, lane, v);
  } else {
    const float s = store_q7_row<EPL>(reinterpret_cast<int8_t*>(out) + (size_t)r * Wd, lane, v);
    if (lane == 0) out_scale[r] = s;
  }
}

// --------------------------------------------------------------------------
// residual update from split-K partial products, fused with the next norm
// --------------------------------------------------------------------------

// x[r] += p_0[r] + ... + p_{S-1}[r] (in split order, in fp32), written back
// (rounded to bf16 with XB); then LayerNorm / conversion / quantisation of
// the updated row, as x now holds it, into out (WRITE = false: the
// residual update only).
template <int EPL, int OUT, bool NORM, bool WRITE, bool XB>
__global__ __launch_bounds__(256) void k_resid_ln(void* __restrict__ x, const float* __restrict__ partials,
                                                  int splits, const float* __restrict__ gamma, int rows, float eps,
                                                  void* __restrict__ out, float* __restrict__ out_scale) {
  using RS = RowShape<EPL>;
  constexpr int Wd = RS::W;
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  float v[EPL];
  load_x_row<EPL, XB>(x, (size_t)r, lane, v);
  // up to 4 partial rows in flight at once, added in split order
  for (int sp0 = 0; sp0 < splits; sp0 += 4) {
    float p[4][EPL];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (sp0 + j < splits) load_f32_row<EPL>(partials + ((size_t)(sp0 + j) * rows + r) * Wd, lane, p[j]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (sp0 + j < splits) {
#pragma unroll
        for (int i = 0; i < EPL; ++i) v[i] += p[j][i];
      }
  }
  store_x_row<EPL, XB>(x, (size_t)r, lane, v);
  if constexpr (WRITE) {
    if constexpr (NORM) layernorm_regs<EPL>(v, gamma, lane, eps);
    if constexpr (OUT == O_F32) {
      store_f32_row<EPL>(reinterpret_cast<float*>(out) + (size_t)r * Wd, lane, v);
    } else if constexpr (OUT == O_BF16) {
      store_bf16_row<EPL>(reinterpret_cast<uint16_t*>(out) + (size_t)r * Wd, lane, v);
    } else {
      const float s = store_q7_row<EPL>(reinterpret_cast<int8_t*>(out) + (size_t)r * Wd, lane, v);
      if (lane == 0) out_scale[r] = s;
    }
  }
}

// --------------------------------------------------------------------------
// final LayerNorm + mean pool + L2 normalisation
// --------------------------------------------------------------------------

// Stage 1: one block per unit (up to POOL_ROWS rows of one text): LayerNorm
// of each row in registers, per-wave column sums, then a fixed-order sum of
// the 4 waves through LDS -> partial[u, :].  No atomics: deterministic.
template <int EPL, bool XB>
__global__ __launch_bounds__(256) void k_pool_partial(const void* __restrict__ x, const float* __restrict__ gamma,
                                                      float eps, const int* __restrict__ off,
                                                      const int* __restrict__ unit_start, int n_texts,
                                                      float* __restrict__ partial) {
  using RS = RowShape<EPL>;
  constexpr int H = RS::W;
  __shared__ float red[4][H];
  const int u = blockIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lo = wave_find(unit_start, n_texts, u);  // text b with unit_start[b] <= u < unit_start[b+1]
  const int r0 = off[lo] + (u - unit_start[lo]) * POOL_ROWS;
  const int r1 = min(r0 + POOL_ROWS, off[lo + 1]);
  float acc[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) acc[i] = 0.f;
  // a wave's rows r0 + w, r0 + w + 4, ...: RB rows' loads in flight at a
  // time, then normalised and added in row order
  constexpr int RB = EPL <= 12 ? 8 : (EPL <= 24 ? 4 : (EPL <= 48 ? 2 : 1));
  for (int rb = r0 + w; rb < r1; rb += 4 * RB) {
    float v[RB][EPL];
#pragma unroll
    for (int k = 0; k < RB; ++k)
      if (rb + 4 * k < r1) load_x_row<EPL, XB>(x, (size_t)(rb + 4 * k), lane, v[k]);
#pragma unroll
    for (int k = 0; k < RB; ++k) {
      if (rb + 4 * k < r1) {  // wave-uniform
        layernorm_regs<EPL>(v[k], gamma, lane, eps);
#pragma unroll
        for (int i = 0; i < EPL; ++i) acc[i] += v[k][i];
      }
    }
  }
#pragma unroll
  for (int c = 0; c < RS::CH; ++c)
#pragma unroll
    for (int e = 0; e < RS::VEC; ++e) red[w][RS::col(c, lane, e)] = acc[c * RS::VEC + e];
  __syncthreads();
  for (int j = threadIdx.x; j < H; j += 256)
    partial[(size_t)u * H + j] = ((red[0][j] + red[1][j]) + red[2][j]) + red[3][j];
}

// Stage 2: one block per text: sum its units in order, divide by the token
// count, divide by max(||e||, 1e-12).
template <int H>
__global__ __launch_bounds__(256) void k_pool_finish(const float* __restrict__ partial, const int* __restrict__ off,
                                                     const int* __restrict__ unit_start, float* __restrict__ out,
                                                     const PackIO* __restrict__ io) {
  constexpr int PER = (H + 255) / 256;
  __shared__ float red[4];
  const int b = blockIdx.x;
  if (io) out = io->out;
  const int u0 = unit_start[b], u1 = unit_start[b + 1];
  const float inv_n = 1.f / (float)(off[b + 1] - off[b]);
  float e[PER];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = threadIdx.x + 256 * i;
    float s = 0.f;
    if (j < H) {
      // 8 units' loads in flight at a time, then added in unit order (the
      // same sum as one unit at a time, without a load latency per unit)
      for (int u = u0; u < u1; u += 8) {
        float t[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) t[k] = u + k < u1 ? partial[(size_t)(u + k) * H + j] : 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (u + k < u1) s += t[k];
      }
    }
    e[i] = s * inv_n;
    ss += (j < H) ? e[i] * e[i] : 0.f;
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float norm = sqrtf(((red[0] + red[1]) + red[2]) + red[3]);
  const float inv = 1.f / fmaxf(norm, 1e-12f);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = threadIdx.x + 256 * i;
    if (j < H) out[(size_t)b * H + j] = e[i] * inv;
  }
}

// --------------------------------------------------------------------------
// launchers
// --------------------------------------------------------------------------

bool row_width_supported(int width) {
  if (width <= 0 || width % 64 != 0) return false;
  switch (width / 64) {
    case 2: case 4: case 8: case 12: case 16: case 24: case 32: case 48: case 64: return true;
    default: return false;
  }
}

#define TTE_EPL_DISPATCH(width, MACRO) \
  switch ((width) / 64) {              \
    case 2: MACRO(2); break;           \
    case 4: MACRO(4); break;           \
    case 8: MACRO(8); break;           \
    case 12: MACRO(12); break;         \
    case 16: MACRO(16); break;         \
    case 24: MACRO(24); break;         \
    case 32: MACRO(32); break;         \
    case 48: MACRO(48); break;         \
    case 64: MACRO(64); break;         \
    default: break;                    \
  }

void launch_embed_ln(int prec, const int32_t* ids, const PackIO* io, int T, const void* table, const float* table_scale,
                     int vocab, const float* gamma, float eps, int H, const int* d_off, int n_texts, void* x,
                     int x_kind, Seg* seg, hipStream_t s) {
  if (T <= 0) return;
  const dim3 grid((T + 3) / 4), block(256);
#define L_EMB(E)                                                                                                      \
  if (prec == P_F32)                                                                                                  \
    launch_timed(k_embed_ln<E, P_F32, false>, grid, block, 0, s, ids, io, T, table, table_scale, vocab, gamma, eps,   \
                 d_off, n_texts, x, seg);                                                                             \
  else if (prec == P_BF16 && x_kind == O_BF16)                                                                        \
    launch_timed(k_embed_ln<E, P_BF16, true>, grid, block, 0, s, ids, io, T, table, table_scale, vocab, gamma, eps,   \
                 d_off, n_texts, x, seg);                                                                             \
  else if (prec == P_BF16)                                                                                            \
    launch_timed(k_embed_ln<E, P_BF16, false>, grid, block, 0, s, ids, io, T, table, table_scale, vocab, gamma, eps,  \
                 d_off, n_texts, x, seg);                                                                             \
  else                                                                                                                \
    launch_timed(k_embed_ln<E, P_I8, false>, grid, block, 0, s, ids, io, T, table, table_scale, vocab, gamma, eps,    \
                 d_off, n_texts, x, seg);
  TTE_EPL_DISPATCH(H, L_EMB)
#undef L_EMB
}

// fp32 x: every output form, with or without the norm; bf16 x: fp32 and
// bf16 outputs only (the bf16 mode has no 7-bit codes).
void launch_ln(const void* x, int x_kind, const float* gamma, int rows, int width, float eps, int out_kind, void* out,
               float* out_scale, hipStream_t s, const PackIO* io) {
  if (rows <= 0) return;
  const dim3 grid((rows + 3) / 4), block(256);
#define L_LN_X(E, NORM)                                                                                              \
  if (x_kind == O_BF16) {                                                                                            \
    if (out_kind == O_F32)                                                                                           \
      launch_timed(k_ln<E, O_F32, NORM, true>, grid, block, 0, s, x, gamma, rows, eps, out, out_scale, io);          \
    else if (out_kind == O_BF16)                                                                                     \
      launch_timed(k_ln<E, O_BF16, NORM, true>, grid, block, 0, s, x, gamma, rows, eps, out, out_scale, io);         \
  } else if (out_kind == O_F32) {                                                                                    \
    launch_timed(k_ln<E, O_F32, NORM, false>, grid, block, 0, s, x, gamma, rows, eps, out, out_scale, io);           \
  } else if (out_kind == O_BF16) {                                                                                   \
    launch_timed(k_ln<E, O_BF16, NORM, false>, grid, block, 0, s, x, gamma, rows, eps, out, out_scale, io);          \
  } else {                                                                                                           \
    launch_timed(k_ln<E, O_I8, NORM, false>, grid, block, 0, s, x, gamma, rows, eps, out, out_scale, io);            \
  }
#define L_LN(E)           \
  if (gamma) {            \
    L_LN_X(E, true)       \
  } else {                \
    L_LN_X(E, false)      \
  }
  TTE_EPL_DISPATCH(width, L_LN)
#undef L_LN
#undef L_LN_X
}

void launch_quant7(const float* x, int rows, int width, int8_t* q, float* scale, hipStream_t s) {
  launch_ln(x, O_F32, nullptr, rows, width, 0.f, O_I8, q, scale, s);
}

// fp32 x: the update alone or with any output form; bf16 x: the update
// alone, or with the norm into bf16 (the forms the bf16 mode runs).
void launch_resid_ln(void* x, int x_kind, const float* partials, int splits, const float* gamma, int rows, int width,
                     float eps, int out_kind, void* out, float* out_scale, hipStream_t s) {
  if (rows <= 0) return;
  const dim3 grid((rows + 3) / 4), block(256);
#define RLN(E, OUT, NORM, WRITE, XB)                                                                               \
  launch_timed(k_resid_ln<E, OUT, NORM, WRITE, XB>, grid, block, 0, s, x, partials, splits, gamma, rows, eps, out, \
               out_scale)
#define L_RLN(E)                                                                     \
  if (x_kind == O_BF16) {                                                            \
    if (out_kind < 0) RLN(E, O_F32, false, false, true);                             \
    else if (gamma && out_kind == O_BF16) RLN(E, O_BF16, true, true, true);          \
  } else if (out_kind < 0) {                                                         \
    RLN(E, O_F32, false, false, false);                                              \
  } else if (gamma) {                                                                \
    if (out_kind == O_F32) RLN(E, O_F32, true, true, false);                         \
    else if (out_kind == O_BF16) RLN(E, O_BF16, true, true, false);                  \
    else RLN(E, O_I8, true, true, false);                                            \
  } else {                                                                           \
    if (out_kind == O_F32) RLN(E, O_F32, false, true, false);                        \
    else if (out_kind == O_BF16) RLN(E, O_BF16, false, true, false);                 \
    else RLN(E, O_I8, false, true, false);                                           \
  }
  TTE_EPL_DISPATCH(width, L_RLN)
#undef L_RLN
#undef RLN
}

void launch_pool(const void* x, int x_kind, const float* gamma, float eps, int H, const int* d_off, const int* d_unit,
                 int n_texts, int n_units, float* partial, float* out, hipStream_t s, const PackIO* io) {
  if (n_texts <= 0) return;
#define L_POOL(E)                                                                                          \
  if (x_kind == O_BF16) k_pool_partial<E, true><<<n_units, 256, 0, s>>>(x, gamma, eps, d_off, d_unit, n_texts, partial); \
  else k_pool_partial<E, false><<<n_units, 256, 0, s>>>(x, gamma, eps, d_off, d_unit, n_texts, partial);   \
  k_pool_finish<E * 64><<<n_texts, 256, 0, s>>>(partial, d_off, d_unit, out, io);
  TTE_EPL_DISPATCH(H, L_POOL)
#undef L_POOL
}

LaunchEvents& next_launch_events() {
  thread_local LaunchEvents e;
  return e;
}

}  // namespace tte
