// Host-side launchers of the gfx950 kernels.  Every launcher assumes its
// arguments were validated by the caller (tte.hip): shapes supported,
// pointers non-null, grids in bounds.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tte {

// P_I4: 4-bit weight codes (two per byte) with a 16-byte record per 128
// inputs of a weight row (block scales and offsets), 7-bit int8 activation
// codes; numbered as the ABI's precisions.
enum Prec { P_F32 = 0, P_BF16 = 1, P_I8 = 2, P_I4 = 3 };
enum OutKind { O_F32 = 0, O_BF16 = 1, O_I8 = 2 };
enum Epi { E_STORE = 0, E_RESID = 1, E_GEGLU = 2, E_QKV = 3, E_PART = 4 };

// Per-token text bounds: seg[t] = {offsets[b], offsets[b+1]} of t's text.
struct Seg {
  int start, end;
};

// Column of token t in a bf16 V^T row: within each aligned group of 32
// tokens, token 16 h + 4 k + r (h < 2, k < 4, r < 4) sits at 8 k + 4 h + r,
// so the 8 keys an attention lane multiplies (4 k .. 4 k + 3 and
// 16 + 4 k .. 16 + 4 k + 3 of a group) are one 16-byte run.  fp32 V^T rows
// are in token order.
__host__ __device__ inline int vt_col_bf16(int t) {
  return (t & ~31) | ((t >> 2) & 3) << 3 | ((t >> 4) & 1) << 2 | (t & 3);
}

// Extra operands of the QKV projection's epilogue: RoPE of the Q and K
// columns (positions from the per-token text bounds) and V written
// transposed, vt[h * 64 + d][col(t)] with row stride vt_stride tokens
// (col = vt_col_bf16 for bf16, t for fp32).
struct QkvOut {
  const Seg* seg;
  const float* cos_tab;
  const float* sin_tab;
  void* vt;
  int vt_stride;
  int hidden;
};

// Pointers of one embedding call kept in device memory, so that a replayed
// graph of the pass reads the call's token ids and writes its output
// wherever the caller's buffers are.  Launchers take it nullable: with
// io == nullptr the kernels use the pointers they are given.
struct PackIO {
  const int32_t* ids;
  float* out;
};

// Row widths (H or I) the row kernels handle: multiples of 64 with
// width/64 in this set.
bool row_width_supported(int width);

// The residual stream x [T, H] is fp32 (x_kind O_F32), or bf16 (O_BF16)
// in the bf16 mode; its updates are added in fp32 and rounded once when
// stored.

// Gather rows of the token table (fp32, bf16, or int8 blocks with fp32
// scales), bias-free LayerNorm with gain `gamma`, write x [T, H] (bf16 x
// with a bf16 table only).  Also writes seg[t] from the device copy of the
// offsets.
void launch_embed_ln(int prec, const int32_t* ids, const PackIO* io, int T, const void* table,
                     const float* table_scale, int vocab, const float* gamma, float eps, int H, const int* d_off,
                     int n_texts, void* x, int x_kind, Seg* seg, hipStream_t s);

// Bias-free LayerNorm (gamma non-null) or plain conversion (gamma null) of
// fp32 rows to fp32 / bf16 / 7-bit int8 codes + row scales; of bf16 rows
// to fp32 / bf16.
void launch_ln(const void* x, int x_kind, const float* gamma, int rows, int width, float eps, int out_kind, void* out,
               float* out_scale, hipStream_t s, const PackIO* io = nullptr);

// Per-row 7-bit quantisation.
void launch_quant7(const float* x, int rows, int width, int8_t* q, float* scale, hipStream_t s);

// Timing of the next kernel this thread launches through launch_timed:
// when set, the kernel is launched with these events recorded as part of
// its dispatch (hipExtLaunchKernel) and the slot is cleared, so its
// measured duration is the kernel's alone, with no separate marker
// packets.  Set by the engine's per-launch profiler.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
LaunchEvents& next_launch_events();

template <typename... KArgs, typename... Args>
inline void launch_timed(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t shmem, hipStream_t s,
                         Args... args) {
  LaunchEvents& ev = next_launch_events();
  if (ev.start) {
    const LaunchEvents e = ev;
    ev = LaunchEvents{};
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, e.start, e.stop, 0u, static_cast<KArgs>(args)...);
  } else {
    kernel<<<grid, block, shmem, s>>>(static_cast<KArgs>(args)...);
  }
}

// C = A * W^T with epilogue; see tte_op_gemm.  Requires N % 128 == 0
// (GEGLU: N % 64 == 0) and K % 128 == 0.  E_RESID adds into fp32 C, or,
// for bf16 operands with out_kind O_BF16, into bf16 C (the sum taken in
// fp32, rounded once).
void launch_gemm(int prec, int epi, const void* A, const float* a_scale, const void* W, const float* w_scale,
                 int M, int N, int K, void* C, int out_kind, hipStream_t s);

// Split-K product for the residual projections: the K range is cut into
// `splits` equal parts (K % (128 * splits / element bytes) == 0) and part s
// writes its fp32 partial product to C + s * M * N.  The partials are summed
// into the residual stream, in split order, by launch_resid_ln.
void launch_gemm_splitk(int prec, const void* A, const float* a_scale, const void* W, const float* w_scale, int M,
                        int N, int K, int splits, float* partials, hipStream_t s);

// Number of K parts (1 .. max_splits) for a residual product M x N x K
// run split (launch_gemm_splitk): enough to fill two blocks per compute
// unit, each part at least 6 K tiles.
int residual_splits(int prec, int M, int N, int K, int max_splits);

// x += partials[0] + ... + partials[splits-1] (in that order), then the
// bias-free LayerNorm (gamma non-null) or plain conversion (gamma null) of
// the new x to out (fp32 / bf16 / 7-bit codes + scales), or no output
// (out_kind < 0).  bf16 x: the update alone, or with the norm into bf16.
// One wave per row.
void launch_resid_ln(void* x, int x_kind, const float* partials, int splits, const float* gamma, int rows, int width,
                     float eps, int out_kind, void* out, float* out_scale, hipStream_t s);

// QKV projection with the RoPE / transposed-V epilogue: writes rotated Q
// and K into qkv [M, 3H] (columns 0 .. 2H-1) and V into qo.vt.  Requires
// the per-token text bounds of the pack in qo.seg.  fill (bf16, the
// latency mode): tiles that fill the chip for one pack on its own.
void launch_gemm_qkv(int prec, const void* A, const float* a_scale, const void* W, const float* w_scale, int M,
                     int K, void* qkv, int out_kind, const QkvOut& qo, hipStream_t s, bool fill = false);

// The same RoPE and V transposition from an unrotated qkv [T, 3H] (for the
// single-kernel attention entry point).
void launch_qkv_prep(int prec, const void* qkv_in, void* qk_out, const QkvOut& qo, int T, hipStream_t s);

// Attention over the packed axis.  qk: [T, 3H] with rotated Q and K in
// columns 0 .. 2H-1; vt: V transposed [H][vt_stride]; o: [T, H].  fp32 or
// bf16 operands.  mean_len: the pack's mean text length (tokens), which
// picks the query block size.  d_off / d_qunit (device, n_texts + 1 each):
// the offsets and the starts of each text's units of ATTN_QUNIT queries
// (prefix sums of ceil(len / ATTN_QUNIT)); with them the 64-query blocks
// are text-aligned units, without them BQ consecutive queries of the pack.
constexpr int ATTN_QUNIT = 64;
void launch_attention(int prec, const void* qk, const void* vt, int vt_stride, void* o, const Seg* seg, int T,
                      int n_heads, int is_global, int window, int mean_len, hipStream_t s, const int* d_off = nullptr,
                      const int* d_qunit = nullptr, int n_texts = 0);

// Cosine-similarity matrix of unit vectors: sim [n, n] = E E^T, E fp32
// [n, dim] row-major, dim % 16 == 0.
void launch_similarity(const float* e, int n, int dim, float* sim, hipStream_t s);

// Final LayerNorm + mean per text + L2.  Units of up to POOL_ROWS rows of
// one text: unit_start[b] .. unit_start[b+1] belong to text b.
constexpr int POOL_ROWS = 32;
void launch_pool(const void* x, int x_kind, const float* gamma, float eps, int H, const int* d_off, const int* d_unit,
                 int n_texts, int n_units, float* partial, float* out, hipStream_t s, const PackIO* io = nullptr);

}  // namespace tte
