// Host-side launchers of the gfx950 kernels.  Every launcher assumes its
// arguments were validated by the caller (tte.hip): shapes supported,
// pointers non-null, grids in bounds.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tte {

enum Prec { P_F32 = 0, P_BF16 = 1, P_I8 = 2 };
enum OutKind { O_F32 = 0, O_BF16 = 1, O_I8 = 2 };
enum Epi { E_STORE = 0, E_RESID = 1, E_GEGLU = 2 };

// Per-token text bounds: seg[t] = {offsets[b], offsets[b+1]} of t's text.
struct Seg {
  int start, end;
};

// Row widths (H or I) the row kernels handle: multiples of 64 with
// width/64 in this set.
bool row_width_supported(int width);

// Gather rows of the token table (fp32, bf16, or int8 blocks with fp32
// scales), bias-free LayerNorm with gain `gamma`, write fp32 x [T, H].
// Also writes seg[t] from the device copy of the offsets.
void launch_embed_ln(int prec, const int32_t* ids, int T, const void* table, const float* table_scale,
                     int vocab, const float* gamma, float eps, int H, const int* d_off, int n_texts, float* x,
                     Seg* seg, hipStream_t s);

// Bias-free LayerNorm (gamma non-null) or plain conversion (gamma null) of
// fp32 rows to fp32 / bf16 / 7-bit int8 codes + row scales.
void launch_ln(const float* x, const float* gamma, int rows, int width, float eps, int out_kind, void* out,
               float* out_scale, hipStream_t s);

// Per-row 7-bit quantisation.
void launch_quant7(const float* x, int rows, int width, int8_t* q, float* scale, hipStream_t s);

// C = A * W^T with epilogue; see tte_op_gemm.  Requires N % 128 == 0
// (GEGLU: N % 64 == 0) and K % 128 == 0.
void launch_gemm(int prec, int epi, const void* A, const float* a_scale, const void* W, const float* w_scale,
                 int M, int N, int K, void* C, int out_kind, hipStream_t s);

// Attention over the packed axis; qkv [T, 3H] -> o [T, H] (fp32 or bf16).
void launch_attention(int prec, const void* qkv, void* o, const Seg* seg, const float* cos_tab,
                      const float* sin_tab, int T, int n_heads, int is_global, int window, hipStream_t s);

// Final LayerNorm + mean per text + L2.  Units of up to POOL_ROWS rows of
// one text: unit_start[b] .. unit_start[b+1] belong to text b.
constexpr int POOL_ROWS = 32;
void launch_pool(const float* x, const float* gamma, float eps, int H, const int* d_off, const int* d_unit,
                 int n_texts, int n_units, float* partial, float* out, hipStream_t s);

}  // namespace tte
