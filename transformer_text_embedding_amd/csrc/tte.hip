// C ABI and engine: configuration checks, workspace carve-up, RoPE tables,
// host-side validation of packs, and the per-layer launch sequence of the
// packed embedding pass (tensai "テキスト埋め込み" page, section 何が動くか:
// embedding, 25 pre-norm layers of attention + GeGLU with the global/local
// schedule, mean pooling and unit length).
//
// Layer structure (the ModernBERT layout the page names): embedding
// LayerNorm; per layer, x += Wo * attn(Wqkv * norm_attn(x)) with no norm on
// layer 0, then x += Wo2 * GeGLU(Wi * norm_mlp(x)); final LayerNorm; mean
// over each text; L2 normalisation.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"
#include "tte.h"

using namespace tte;

namespace {

thread_local std::string g_err;

// Diagnostics switched on from the environment (read once per process):
// TTE_LOG=1 writes one stderr line per model creation, per pass and per
// error; TTE_DEBUG=1 adds host-side checks around every pass, each of which
// waits for the stream (slow; for finding faults, not for timing): token
// ids in [0, vocab) (the normal path clamps them on the device), guard
// words after every workspace region intact, and the outputs finite (pooled
// vectors of unit length).
bool env_on(const char* name) {
  const char* v = std::getenv(name);
  return v && v[0] && std::strcmp(v, "0") != 0;
}
bool log_on() {
  static const bool on = env_on("TTE_LOG");
  return on;
}
bool debug_on() {
  static const bool on = env_on("TTE_DEBUG");
  return on;
}

__attribute__((format(printf, 1, 2))) void log_line(const char* fmt, ...) {
  if (!log_on()) return;
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  std::fprintf(stderr, "[tte] %s\n", buf);
}

tte_status fail(tte_status s, const std::string& msg) {
  g_err = msg;
  log_line("error %d: %s", (int)s, msg.c_str());
  return s;
}

// TTE_DEBUG: bytes of the guard after each workspace region, and its fill
constexpr size_t GUARD_BYTES = 256;
constexpr unsigned char GUARD_FILL = 0xA5;
constexpr int MAX_GUARDS = 16;

size_t al(size_t v) { return (v + 255) & ~size_t(255); }

// most K parts of a split residual product (TTE_FLAG_SPLIT_K)
constexpr int MAX_SPLITS = 4;

struct Layout {
  size_t x, xa, ascale, qkv, vt, o, y, kpart, seg, off, partial, cosg, sing, cosl, sinl, total;
  int max_units;
  int vt_stride;
  size_t guard[MAX_GUARDS];  // TTE_DEBUG: a guard after every region
  int n_guards;
};

int act_bytes(int prec) { return prec == TTE_BF16 ? 2 : 4; }

// The residual stream is held in bf16 in the bf16 mode (every update is
// added in fp32 and rounded once), in fp32 otherwise.
int x_kind(int prec) { return prec == TTE_BF16 ? O_BF16 : O_F32; }

Layout layout_of(const tte_config& c) {
  Layout L{};
  const size_t T = (size_t)c.max_tokens, H = (size_t)c.hidden, I = (size_t)c.intermediate;
  const size_t ab = (size_t)act_bytes(c.precision);
  L.max_units = c.max_tokens / POOL_ROWS + c.max_texts + 1;
  size_t p = 0;
  const bool guards = debug_on();
  auto take = [&](size_t bytes) {
    const size_t at = p;
    p += al(bytes);
    if (guards && L.n_guards < MAX_GUARDS) {
      L.guard[L.n_guards++] = p;
      p += GUARD_BYTES;
    }
    return at;
  };
  L.x = take(T * H * ab);  // the residual stream: bf16 in the bf16 mode, else fp32
  L.xa = take(c.precision >= TTE_INT8 ? T * (H > I ? H : I) : T * H * ab);
  L.ascale = take(T * 4);
  L.qkv = take(T * 3 * H * ab);
  // V transposed, [H][vt_stride]: 64 tokens of slack so a key tile that
  // starts at the last token stays inside the buffer
  L.vt_stride = (int)((T + 64 + 7) / 8 * 8);
  L.vt = take(H * (size_t)L.vt_stride * ab);
  L.o = take(T * H * ab);
  L.y = take(T * I * ab);
  // split-K partials of the residual products
  L.kpart = take(c.flags & TTE_FLAG_SPLIT_K ? (size_t)MAX_SPLITS * T * H * 4 : 0);
  L.seg = take(T * sizeof(Seg));
  // the call's PackIO, then its offsets, pool-unit starts and attention
  // query-unit starts back to back
  L.off = take(sizeof(PackIO) + 3 * ((size_t)c.max_texts + 1) * 4);
  L.partial = take((size_t)L.max_units * H * 4);
  const size_t rope = (size_t)c.max_text_len * 32 * 4;
  L.cosg = take(rope);
  L.sing = take(rope);
  L.cosl = take(rope);
  L.sinl = take(rope);
  L.total = p;
  return L;
}

bool check_config(const tte_config* c, std::string* why) {
  auto bad = [&](const char* m) {
    *why = m;
    return false;
  };
  if (!c) return bad("config is NULL");
  if (c->precision < TTE_FP32 || c->precision > TTE_INT4)
    return bad("precision must be TTE_FP32, TTE_BF16, TTE_INT8 or TTE_INT4");
  if (c->precision == TTE_INT4 && (c->hidden % 256 != 0 || c->intermediate % 256 != 0))
    return bad("TTE_INT4 needs hidden and intermediate multiples of 256 (whole 4-bit super-blocks)");
  if (c->vocab <= 0 || c->n_layers <= 0 || c->n_heads <= 0) return bad("vocab, n_layers and n_heads must be positive");
  if (c->head_dim != 64) return bad("head_dim must be 64");
  if (c->hidden != c->n_heads * c->head_dim) return bad("hidden must equal n_heads * head_dim");
  if (c->hidden % 128 != 0 || !row_width_supported(c->hidden))
    return bad("hidden must be a multiple of 128 with hidden/64 in {2,4,8,12,16,24,32,48,64}");
  if (c->intermediate <= 0 || c->intermediate % 128 != 0 || !row_width_supported(c->intermediate))
    return bad("intermediate must be a multiple of 128 with intermediate/64 in {2,4,8,12,16,24,32,48,64}");
  if (c->global_every <= 0) return bad("global_every must be positive");
  if (c->window < 0) return bad("window must be >= 0");
  if (!(c->ln_eps > 0.f)) return bad("ln_eps must be > 0");
  if (!(c->rope_base_global > 0.f) || !(c->rope_base_local > 0.f)) return bad("RoPE bases must be > 0");
  if (c->max_tokens <= 0 || c->max_text_len <= 0 || c->max_texts <= 0)
    return bad("max_tokens, max_text_len and max_texts must be positive");
  if (c->max_tokens > (1 << 24)) return bad("max_tokens above 2^24");
  if (c->flags & ~int32_t(TTE_FLAG_SPLIT_K | TTE_FLAG_GRAPH)) return bad("unknown flag");
  return true;
}

// The GEMM kernels address a W row as a 32-bit byte offset from W's base
// (row * row bytes + the K tile's offset): every byte of W must lie below
// 2^32.  n_w = rows of W (2N for the GeGLU product).
bool weight_offsets_fit(int precision, int64_t n_w, int64_t K) {
  const int64_t bytes_per_k = precision == TTE_FP32 ? 4 : precision == TTE_BF16 ? 2 : 1;
  const int64_t row = precision == TTE_INT4 ? K / 2 : K * bytes_per_k;
  return n_w * row <= (int64_t)UINT32_MAX;
}

tte_status check_pack(const tte_config& c, int32_t n_tokens, const int32_t* h_off, int32_t n_texts) {
  if (n_texts < 0 || n_tokens < 0) return fail(TTE_E_INVALID, "n_texts and n_tokens must be >= 0");
  if (n_texts == 0) {
    if (n_tokens != 0) return fail(TTE_E_INVALID, "n_tokens must be 0 when n_texts is 0");
    return TTE_OK;
  }
  if (!h_off) return fail(TTE_E_INVALID, "h_offsets is NULL");
  if (n_texts > c.max_texts) return fail(TTE_E_INVALID, "n_texts exceeds max_texts");
  if (n_tokens > c.max_tokens) return fail(TTE_E_INVALID, "n_tokens exceeds max_tokens");
  if (h_off[0] != 0) return fail(TTE_E_INVALID, "offsets[0] must be 0");
  for (int b = 0; b < n_texts; ++b) {
    const int64_t len = (int64_t)h_off[b + 1] - h_off[b];
    if (len <= 0) return fail(TTE_E_INVALID, "offsets must be strictly increasing (empty text at " + std::to_string(b) + ")");
    if (len > c.max_text_len) return fail(TTE_E_INVALID, "text " + std::to_string(b) + " is longer than max_text_len");
  }
  if (h_off[n_texts] != n_tokens) return fail(TTE_E_INVALID, "offsets[n_texts] must equal n_tokens");
  return TTE_OK;
}

}  // namespace

struct tte_model {
  tte_config cfg;
  tte_weights w;
  std::vector<tte_layer_weights> layers;
  Layout L;
  uint8_t* ws;
  int device;
  // carved workspace
  void* x;  // residual stream [T, H], format x_kind(precision)
  void* xa;
  float* ascale;
  void* qkv;
  void* vt;
  void* o;
  void* y;
  float* kpart;
  Seg* seg;
  PackIO* d_io;  // the call's ids / output pointers (read by graph replays)
  int* d_off;
  int* d_unit;   // d_off + n_texts + 1 of the last upload
  int* d_qunit;  // d_off + 2 (n_texts + 1): starts of each text's 64-query attention units
  float* partial;
  const float *cosg, *sing, *cosl, *sinl;
  // pinned staging for the per-call offsets upload: a ring of slots, each
  // reused only after the copy that read it has completed
  int* h_stage;
  hipEvent_t stage_ev[8];
  bool stage_pending[8];
  int stage_next;
  // profiling
  bool prof_on;
  uint32_t prof_mask;
  std::vector<hipEvent_t> ev;
  std::vector<int> ev_cls;
  int ev_used;
  bool ev_overflow;
  // TTE_FLAG_GRAPH: pack shapes seen, and the graphs of those seen twice
  struct GraphEntry {
    int kind, T, B, units;
    hipGraphExec_t exec;  // null until the shape's second call
    hipEvent_t done;      // recorded after each replay: the last one has ended once it completes
    bool failed;          // capture did not succeed: run eagerly
    uint64_t used;
  };
  std::vector<GraphEntry> graphs;
  uint64_t graph_clock;
  int64_t graph_replays;
};

namespace {

// An event pair around the launch of one kernel class.  A class that is one
// kernel takes its pair as part of that kernel's dispatch
// (next_launch_events), so its duration is the kernel's alone; pooling (two
// kernels) records the pair as marker packets on the stream around them.
struct ProfScope {
  tte_model* m;
  hipStream_t s;
  int idx;
  bool in_dispatch;
  ProfScope(tte_model* m_, int cls, hipStream_t s_) : m(m_), s(s_), idx(-1), in_dispatch(false) {
    if (!m->prof_on || !(m->prof_mask & (1u << cls))) return;
    if (2 * (m->ev_used + 1) > (int)m->ev.size()) {
      m->ev_overflow = true;
      return;
    }
    idx = m->ev_used++;
    m->ev_cls[idx] = cls;
    in_dispatch = cls != TTE_K_POOL;
    if (in_dispatch) next_launch_events() = LaunchEvents{m->ev[2 * idx], m->ev[2 * idx + 1]};
    else (void)hipEventRecord(m->ev[2 * idx], s);
  }
  ~ProfScope() {
    if (idx < 0) return;
    if (!in_dispatch) {
      (void)hipEventRecord(m->ev[2 * idx + 1], s);
      return;
    }
    LaunchEvents& e = next_launch_events();
    if (e.start) {  // nothing was launched (an empty pack): an empty pair
      (void)hipEventRecord(e.start, s);
      (void)hipEventRecord(e.stop, s);
      e = LaunchEvents{};
    }
  }
};

tte_status hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return TTE_OK;
  return fail(TTE_E_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

// Copies the call's PackIO, offsets and pool-unit starts into the
// workspace in one stream-ordered copy, from pinned staging that is reused
// only once the previous copy from it is done.  Sets m->d_unit.
constexpr int STAGE_SLOTS = 8;

size_t stage_ints(const tte_config& c) { return sizeof(PackIO) / 4 + 3 * ((size_t)c.max_texts + 1); }

tte_status upload_pack(tte_model* m, const int32_t* h_off, int n_texts, int* n_units, hipStream_t s,
                       const int32_t* d_ids = nullptr, float* d_out = nullptr) {
  const int slot = m->stage_next;
  m->stage_next = (slot + 1) % STAGE_SLOTS;
  if (m->stage_pending[slot]) {
    tte_status st = hip_check(hipEventSynchronize(m->stage_ev[slot]), "hipEventSynchronize");
    if (st != TTE_OK) return st;
    m->stage_pending[slot] = false;
  }
  int* base = m->h_stage + (size_t)slot * stage_ints(m->cfg);
  const PackIO io{d_ids, d_out};
  std::memcpy(base, &io, sizeof(PackIO));
  int* so = base + sizeof(PackIO) / 4;
  int* su = so + (n_texts + 1);
  int* sq = su + (n_texts + 1);
  std::memcpy(so, h_off, sizeof(int) * (size_t)(n_texts + 1));
  su[0] = 0;
  sq[0] = 0;
  for (int b = 0; b < n_texts; ++b) {
    const int len = h_off[b + 1] - h_off[b];
    su[b + 1] = su[b] + (len + POOL_ROWS - 1) / POOL_ROWS;
    sq[b + 1] = sq[b] + (len + ATTN_QUNIT - 1) / ATTN_QUNIT;
  }
  *n_units = su[n_texts];
  m->d_unit = m->d_off + (n_texts + 1);
  m->d_qunit = m->d_off + 2 * (n_texts + 1);
  const size_t bytes = sizeof(PackIO) + sizeof(int) * 3 * (size_t)(n_texts + 1);
  tte_status st = hip_check(hipMemcpyAsync(m->d_io, base, bytes, hipMemcpyHostToDevice, s), "hipMemcpyAsync(offsets)");
  if (st != TTE_OK) return st;
  st = hip_check(hipEventRecord(m->stage_ev[slot], s), "hipEventRecord");
  if (st != TTE_OK) return st;
  m->stage_pending[slot] = true;
  return TTE_OK;
}

// Per-token text bounds from the device offsets (used by the attention
// entry point; the full pass gets them from the embedding kernel).
__global__ void k_seg(const int* __restrict__ off, int n_texts, int T, Seg* __restrict__ seg) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  int lo = 0, hi = n_texts;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= t) lo = mid; else hi = mid;
  }
  seg[t] = Seg{off[lo], off[lo + 1]};
}

// bf16 V^T rows from the attention's column order (vt_col_bf16) to token
// order: out[r][t] = vt[r][col(t)] for r < rows, t < T.
__global__ void k_vt_tokens(const uint16_t* __restrict__ vt, int stride, uint16_t* __restrict__ out, int T, int rows) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long)rows * T) return;
  const int r = (int)(i / T), t = (int)(i % T);
  out[i] = vt[(size_t)r * stride + vt_col_bf16(t)];
}

// The launch sequence of one pass over an uploaded pack.  The output is
// either the pooled unit vectors (d_out [B, H]) or, with d_tok, the
// per-token states after the final LayerNorm ([T, H]); d_states receives
// the residual stream after the embedding norm and each of the first n_run
// layers.  With io non-null the embedding and output kernels take the ids
// and output pointers from it (device memory) instead of d_ids / d_out /
// d_tok.
void enqueue_pass(tte_model* m, const int32_t* d_ids, const PackIO* io, int32_t T, int32_t B, int n_units,
                  float* d_out, float* d_states, int n_run, float* d_tok, hipStream_t s) {
  const tte_config& c = m->cfg;
  const int P = c.precision, H = c.hidden, I = c.intermediate, nh = c.n_heads;
  const int act = P == TTE_BF16 ? O_BF16 : O_F32;  // format of qkv / o / y
  const int xk = x_kind(P);                          // format of the residual stream
  // a trace copies x (converted to fp32 if it is bf16)
  auto dump = [&](int k) {
    float* dst = d_states + (size_t)k * T * H;
    if (xk == O_F32) (void)hipMemcpyAsync(dst, m->x, (size_t)T * H * 4, hipMemcpyDeviceToDevice, s);
    else launch_ln(m->x, xk, nullptr, T, H, 0.f, O_F32, dst, nullptr, s);
  };
  {
    ProfScope ps(m, TTE_K_EMBED, s);
    launch_embed_ln(P == TTE_INT4 ? TTE_INT8 : P, d_ids, io, T, m->w.tok_emb, m->w.tok_emb_scale, c.vocab,
                    m->w.emb_norm, c.ln_eps, H, m->d_off, B, m->x, xk, m->seg, s);
  }
  if (d_states) dump(0);

  // With TTE_FLAG_SPLIT_K the residual products of a short pack run split-K
  // (their H-wide outputs give fewer tiles than the compute units can hold);
  // the partial products are added to the residual stream, in part order,
  // by the next norm kernel.
  const bool split = (c.flags & TTE_FLAG_SPLIT_K) != 0;
  const int o_splits = split ? residual_splits(P, T, H, H, MAX_SPLITS) : 1;
  const int o2_splits = split ? residual_splits(P, T, H, I, MAX_SPLITS) : 1;
  bool pending = false;  // x still lacks the partials of the last down-projection
  const bool integer = P == TTE_INT8 || P == TTE_INT4;  // 7-bit activation codes into the weight products
  const int in_fmt = integer ? O_I8 : act;
  for (int l = 0; l < n_run; ++l) {
    const tte_layer_weights& LW = m->layers[l];
    const int glob = (l % c.global_every) == 0;
    // attention sub-layer input: no norm on layer 0, so the product reads
    // x itself where x is already in the operand format
    const void* a_in = m->xa;
    if (l == 0 && xk == in_fmt) {
      a_in = m->x;
    } else if (pending) {
      ProfScope ps(m, TTE_K_NORM, s);
      launch_resid_ln(m->x, xk, m->kpart, o2_splits, LW.attn_norm, T, H, c.ln_eps, in_fmt, m->xa, m->ascale, s);
      pending = false;
    } else {
      ProfScope ps(m, integer && l == 0 ? TTE_K_QUANT : TTE_K_NORM, s);
      launch_ln(m->x, xk, l == 0 ? nullptr : LW.attn_norm, T, H, c.ln_eps, in_fmt, m->xa, m->ascale, s);
    }
    {
      ProfScope ps(m, TTE_K_GEMM_QKV, s);
      const QkvOut qo{m->seg, glob ? m->cosg : m->cosl, glob ? m->sing : m->sinl, m->vt, m->L.vt_stride, H};
      launch_gemm_qkv(P, a_in, m->ascale, LW.wqkv, LW.wqkv_scale, T, H, m->qkv, act, qo, s, split);
    }
    {
      ProfScope ps(m, glob ? TTE_K_ATTN_GLOBAL : TTE_K_ATTN_LOCAL, s);
      launch_attention(P == TTE_BF16 ? P_BF16 : P_F32, m->qkv, m->vt, m->L.vt_stride, m->o, m->seg, T, nh, glob,
                       c.window, T / B, s, m->d_off, m->d_qunit, B);
    }
    const void* o_in = m->o;
    if (integer) {
      ProfScope ps(m, TTE_K_QUANT, s);
      launch_quant7(reinterpret_cast<const float*>(m->o), T, H, reinterpret_cast<int8_t*>(m->xa), m->ascale, s);
      o_in = m->xa;
    }
    {
      ProfScope ps(m, TTE_K_GEMM_O, s);
      if (o_splits > 1) launch_gemm_splitk(P, o_in, m->ascale, LW.wo, LW.wo_scale, T, H, H, o_splits, m->kpart, s);
      else launch_gemm(P, E_RESID, o_in, m->ascale, LW.wo, LW.wo_scale, T, H, H, m->x, xk, s);
    }
    {
      ProfScope ps(m, TTE_K_NORM, s);
      if (o_splits > 1)
        launch_resid_ln(m->x, xk, m->kpart, o_splits, LW.mlp_norm, T, H, c.ln_eps, in_fmt, m->xa, m->ascale, s);
      else launch_ln(m->x, xk, LW.mlp_norm, T, H, c.ln_eps, in_fmt, m->xa, m->ascale, s);
    }
    {
      ProfScope ps(m, TTE_K_GEMM_GEGLU, s);
      launch_gemm(P, E_GEGLU, m->xa, m->ascale, LW.wi, LW.wi_scale, T, I, H, m->y, act, s);
    }
    const void* y_in = m->y;
    if (integer) {
      ProfScope ps(m, TTE_K_QUANT, s);
      launch_quant7(reinterpret_cast<const float*>(m->y), T, I, reinterpret_cast<int8_t*>(m->xa), m->ascale, s);
      y_in = m->xa;
    }
    {
      ProfScope ps(m, TTE_K_GEMM_O2, s);
      if (o2_splits > 1) {
        launch_gemm_splitk(P, y_in, m->ascale, LW.wo2, LW.wo2_scale, T, H, I, o2_splits, m->kpart, s);
        pending = true;
      } else {
        launch_gemm(P, E_RESID, y_in, m->ascale, LW.wo2, LW.wo2_scale, T, H, I, m->x, xk, s);
      }
    }
    if (pending && (d_states || l + 1 == n_run)) {
      // a trace copies x, and pooling reads it: apply the partials now
      ProfScope ps(m, TTE_K_NORM, s);
      launch_resid_ln(m->x, xk, m->kpart, o2_splits, nullptr, T, H, c.ln_eps, -1, nullptr, nullptr, s);
      pending = false;
    }
    if (d_states) dump(l + 1);
  }
  if (n_run == c.n_layers && d_tok) {
    ProfScope ps(m, TTE_K_NORM, s);
    launch_ln(m->x, xk, m->w.final_norm, T, H, c.ln_eps, O_F32, d_tok, nullptr, s, io);
  } else if (n_run == c.n_layers) {
    ProfScope ps(m, TTE_K_POOL, s);
    launch_pool(m->x, xk, m->w.final_norm, c.ln_eps, H, m->d_off, m->d_unit, B, n_units, m->partial, d_out, s, io);
  }
}

constexpr size_t MAX_GRAPHS = 64;

// Releases a captured graph once its last replay has ended: waits on the
// event recorded behind that replay on its stream (no other stream is
// waited for).  The graph is released even if the wait reports an error.
tte_status release_graph(tte_model::GraphEntry& g) {
  tte_status st = TTE_OK;
  if (g.done) {
    st = hip_check(hipEventSynchronize(g.done), "hipEventSynchronize(graph replay)");
    (void)hipEventDestroy(g.done);
    g.done = nullptr;
  }
  if (g.exec) {
    const tte_status d = hip_check(hipGraphExecDestroy(g.exec), "hipGraphExecDestroy");
    if (st == TTE_OK) st = d;
    g.exec = nullptr;
  }
  return st;
}

// TTE_FLAG_GRAPH: the entry of a pack shape (inserted at its first call,
// the least recently used one dropped beyond MAX_GRAPHS).  Returns null if
// dropping the old entry failed (the error is in tte_last_error).
tte_model::GraphEntry* graph_entry(tte_model* m, int kind, int T, int B, int units, bool* fresh) {
  *fresh = false;
  for (auto& g : m->graphs)
    if (g.kind == kind && g.T == T && g.B == B && g.units == units) return &g;
  if (m->graphs.size() >= MAX_GRAPHS) {
    size_t lru = 0;
    for (size_t i = 1; i < m->graphs.size(); ++i)
      if (m->graphs[i].used < m->graphs[lru].used) lru = i;
    // an earlier replay of it may still run on the stream it was launched on
    const tte_status st = release_graph(m->graphs[lru]);
    m->graphs.erase(m->graphs.begin() + lru);
    if (st != TTE_OK) return nullptr;
  }
  m->graphs.push_back(tte_model::GraphEntry{kind, T, B, units, nullptr, nullptr, false, ++m->graph_clock});
  *fresh = true;
  return &m->graphs.back();
}

// TTE_DEBUG, before a pass: the pack's token ids, read back (the stream
// waits), must lie in [0, vocab).
tte_status debug_check_ids(const tte_model* m, const int32_t* d_ids, int32_t T, hipStream_t s) {
  std::vector<int32_t> ids((size_t)T);
  tte_status st = hip_check(hipMemcpyAsync(ids.data(), d_ids, sizeof(int32_t) * (size_t)T, hipMemcpyDeviceToHost, s),
                            "hipMemcpyAsync(ids)");
  if (st == TTE_OK) st = hip_check(hipStreamSynchronize(s), "hipStreamSynchronize");
  if (st != TTE_OK) return st;
  for (int32_t t = 0; t < T; ++t)
    if (ids[t] < 0 || ids[t] >= m->cfg.vocab)
      return fail(TTE_E_INVALID, "TTE_DEBUG: token id " + std::to_string(ids[t]) + " at index " + std::to_string(t) +
                                     " is outside [0, vocab)");
  return TTE_OK;
}

// TTE_DEBUG, after a pass: the stream's work completed without error, every
// workspace guard still holds its fill, and the outputs are finite (pooled
// vectors of unit length, unless all zero).
tte_status debug_check_after(const tte_model* m, hipStream_t s, int32_t T, int32_t B, const float* d_out,
                             const float* d_tok) {
  tte_status st = hip_check(hipStreamSynchronize(s), "TTE_DEBUG: the pass");
  if (st != TTE_OK) return st;
  unsigned char g[GUARD_BYTES];
  for (int i = 0; i < m->L.n_guards; ++i) {
    st = hip_check(hipMemcpy(g, m->ws + m->L.guard[i], GUARD_BYTES, hipMemcpyDeviceToHost), "hipMemcpy(guard)");
    if (st != TTE_OK) return st;
    for (size_t k = 0; k < GUARD_BYTES; ++k)
      if (g[k] != GUARD_FILL)
        return fail(TTE_E_DEVICE, "TTE_DEBUG: workspace guard " + std::to_string(i) + " overwritten at byte " +
                                      std::to_string(k));
  }
  const int H = m->cfg.hidden;
  const bool pooled = d_out != nullptr;
  const float* src = pooled ? d_out : d_tok;
  if (!src) return TTE_OK;
  const size_t rows = (size_t)(pooled ? B : T);
  std::vector<float> v(rows * (size_t)H);
  st = hip_check(hipMemcpy(v.data(), src, v.size() * 4, hipMemcpyDeviceToHost), "hipMemcpy(out)");
  if (st != TTE_OK) return st;
  for (size_t r = 0; r < rows; ++r) {
    double ss = 0.0;
    for (int j = 0; j < H; ++j) {
      const float x = v[r * H + j];
      if (!std::isfinite(x))
        return fail(TTE_E_DEVICE, "TTE_DEBUG: output row " + std::to_string(r) + " is not finite");
      ss += (double)x * x;
    }
    if (pooled && ss > 0.0 && std::fabs(std::sqrt(ss) - 1.0) > 1e-3)
      return fail(TTE_E_DEVICE, "TTE_DEBUG: output row " + std::to_string(r) + " is not of unit length");
  }
  return TTE_OK;
}

// Validates and uploads a pack, then runs the pass: eagerly, or with
// TTE_FLAG_GRAPH from the graph of the pack's shape (captured at the
// shape's second call).
tte_status run_pass(tte_model* m, const int32_t* d_ids, int32_t T, const int32_t* h_off, int32_t B, float* d_out,
                    float* d_states, int32_t n_dump, void* stream, float* d_tok = nullptr) {
  if (!m) return fail(TTE_E_INVALID, "model is NULL");
  const tte_config& c = m->cfg;
  tte_status st = check_pack(c, T, h_off, B);
  if (st != TTE_OK) return st;
  if (B == 0) return TTE_OK;
  if (!d_ids) return fail(TTE_E_INVALID, "d_token_ids is NULL");
  if (d_states) {
    if (n_dump < 0 || n_dump > c.n_layers) return fail(TTE_E_INVALID, "n_dump must be in [0, n_layers]");
  } else {
    n_dump = -1;
  }
  const int n_run = (d_states && n_dump < c.n_layers) ? n_dump : c.n_layers;
  if (n_run == c.n_layers && !d_out && !d_tok) return fail(TTE_E_INVALID, "d_out is NULL");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  st = hip_check(hipSetDevice(m->device), "hipSetDevice");
  if (st != TTE_OK) return st;
  (void)hipGetLastError();
  const bool debug = debug_on();
  const bool graph = (c.flags & TTE_FLAG_GRAPH) && !d_states && s != nullptr && !m->prof_on && !debug;
  if (debug) {
    st = debug_check_ids(m, d_ids, T, s);
    if (st != TTE_OK) return st;
  }
  int n_units = 0;
  st = upload_pack(m, h_off, B, &n_units, s, graph ? d_ids : nullptr, graph ? (d_tok ? d_tok : d_out) : nullptr);
  if (st != TTE_OK) return st;
  const PackIO* io = graph ? m->d_io : nullptr;
  if (graph) {
    bool fresh = false;
    tte_model::GraphEntry* e = graph_entry(m, d_tok ? 1 : 0, T, B, n_units, &fresh);
    if (!e) return TTE_E_DEVICE;
    e->used = ++m->graph_clock;
    if (!fresh && !e->exec && !e->failed) {
      // second call of this shape: record the sequence (nothing runs while
      // the stream captures) and instantiate it
      hipGraph_t g = nullptr;
      hipError_t err = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
      if (err == hipSuccess) {
        enqueue_pass(m, nullptr, io, T, B, n_units, nullptr, nullptr, n_run, d_tok ? d_tok : nullptr, s);
        err = hipStreamEndCapture(s, &g);
        if (err == hipSuccess) err = hipGraphInstantiate(&e->exec, g, nullptr, nullptr, 0);
        if (g) (void)hipGraphDestroy(g);
        if (err == hipSuccess) err = hipEventCreateWithFlags(&e->done, hipEventDisableTiming);
      }
      (void)hipGetLastError();
      if (err != hipSuccess) {
        if (e->exec) (void)hipGraphExecDestroy(e->exec);
        e->exec = nullptr;
        e->done = nullptr;
        e->failed = true;  // this shape runs eagerly from now on
      }
    }
    if (e->exec) {
      ++m->graph_replays;
      log_line("pass: %d tokens, %d texts, %d pool units, graph replay, stream %p", T, B, n_units, (void*)s);
      st = hip_check(hipGraphLaunch(e->exec, s), "hipGraphLaunch");
      if (st != TTE_OK) return st;
      return hip_check(hipEventRecord(e->done, s), "hipEventRecord(graph replay)");
    }
  }
  log_line("pass: %d tokens, %d texts, %d pool units, %d layers%s, %s output, stream %p", T, B, n_units, n_run,
           d_states ? " (states dumped)" : "", d_tok ? "per-token" : "pooled", (void*)s);
  enqueue_pass(m, d_ids, io, T, B, n_units, d_out, d_states, n_run, d_tok, s);
  st = hip_check(hipGetLastError(), "kernel launch");
  if (st == TTE_OK && debug) st = debug_check_after(m, s, T, B, n_run == c.n_layers ? d_out : nullptr, n_run == c.n_layers ? d_tok : nullptr);
  return st;
}

// --------------------------------------------------------------------------
// Allocation-free pooling (tte_op_pool_static): its scratch -- the pack's
// offsets and pool-unit starts, then the per-unit partial sums -- lives in a
// file-scope device array that each GPU holds from the library's load until
// the process ends.  In host code `scratch` names a host-side stand-in, not
// device memory: every host use goes through the address hipGetSymbolAddress
// returns for the current device (scratch_on), never the array's name.
// --------------------------------------------------------------------------

constexpr size_t STATIC_SCRATCH_BYTES = size_t(8) << 20;  // 8 MiB per GPU
constexpr int STATIC_SCRATCH_DEVICES = 64;

}  // namespace

static __device__ __align__(256) uint8_t scratch[STATIC_SCRATCH_BYTES];

namespace {

std::once_flag g_scratch_once[STATIC_SCRATCH_DEVICES];
uint8_t* g_scratch_ptr[STATIC_SCRATCH_DEVICES];
hipError_t g_scratch_err[STATIC_SCRATCH_DEVICES];

// Device address of `scratch` on `device`, looked up once per device; the
// caller has made `device` current (each GPU holds its own copy of the array
// at its own address).
tte_status scratch_on(int device, uint8_t** out) {
  if (device < 0 || device >= STATIC_SCRATCH_DEVICES)
    return fail(TTE_E_UNSUPPORTED, "static scratch: device index above 63");
  std::call_once(g_scratch_once[device], [device] {
    void* p = nullptr;
    g_scratch_err[device] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[device] = reinterpret_cast<uint8_t*>(p);
  });
  if (g_scratch_err[device] != hipSuccess || !g_scratch_ptr[device])
    return fail(TTE_E_DEVICE, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(g_scratch_err[device]));
  *out = g_scratch_ptr[device];
  return TTE_OK;
}

// Offsets and pool-unit starts of a pack, copied to d_dst through the
// model's pinned staging ring (one stream-ordered copy).
tte_status stage_offsets_to(tte_model* m, const int32_t* h_off, int n_texts, int n_units, void* d_dst,
                            hipStream_t s) {
  const int slot = m->stage_next;
  m->stage_next = (slot + 1) % STAGE_SLOTS;
  if (m->stage_pending[slot]) {
    tte_status st = hip_check(hipEventSynchronize(m->stage_ev[slot]), "hipEventSynchronize");
    if (st != TTE_OK) return st;
    m->stage_pending[slot] = false;
  }
  int* so = m->h_stage + (size_t)slot * stage_ints(m->cfg);
  int* su = so + (n_texts + 1);
  std::memcpy(so, h_off, sizeof(int) * (size_t)(n_texts + 1));
  su[0] = 0;
  for (int b = 0; b < n_texts; ++b) su[b + 1] = su[b] + (h_off[b + 1] - h_off[b] + POOL_ROWS - 1) / POOL_ROWS;
  (void)n_units;
  tte_status st = hip_check(hipMemcpyAsync(d_dst, so, sizeof(int) * 2 * (size_t)(n_texts + 1), hipMemcpyHostToDevice, s),
                            "hipMemcpyAsync(offsets)");
  if (st != TTE_OK) return st;
  st = hip_check(hipEventRecord(m->stage_ev[slot], s), "hipEventRecord");
  if (st != TTE_OK) return st;
  m->stage_pending[slot] = true;
  return TTE_OK;
}

}  // namespace

extern "C" {

const char* tte_last_error(void) { return g_err.c_str(); }

tte_status tte_workspace_size(const tte_config* cfg, size_t* bytes) {
  std::string why;
  if (!check_config(cfg, &why)) return fail(TTE_E_INVALID, why);
  if (!bytes) return fail(TTE_E_INVALID, "bytes is NULL");
  *bytes = layout_of(*cfg).total;
  return TTE_OK;
}

tte_status tte_check_pack(const tte_config* cfg, int32_t n_tokens, const int32_t* h_offsets, int32_t n_texts) {
  std::string why;
  if (!check_config(cfg, &why)) return fail(TTE_E_INVALID, why);
  return check_pack(*cfg, n_tokens, h_offsets, n_texts);
}

tte_status tte_create(const tte_config* cfg, const tte_weights* w, void* d_workspace, size_t workspace_bytes,
                      tte_model** out) {
  std::string why;
  if (!check_config(cfg, &why)) return fail(TTE_E_INVALID, why);
  if (!w || !out) return fail(TTE_E_INVALID, "weights or out is NULL");
  *out = nullptr;
  const tte_config& c = *cfg;
  const bool q = c.precision == TTE_INT8 || c.precision == TTE_INT4;
  if (!w->tok_emb || !w->emb_norm || !w->final_norm || !w->layers || (q && !w->tok_emb_scale))
    return fail(TTE_E_INVALID, "a required weight pointer is NULL");
  for (int l = 0; l < c.n_layers; ++l) {
    const tte_layer_weights& L = w->layers[l];
    if (!L.wqkv || !L.wo || !L.wi || !L.wo2 || !L.mlp_norm || (l > 0 && !L.attn_norm))
      return fail(TTE_E_INVALID, "layer " + std::to_string(l) + ": a required weight pointer is NULL");
    if (q && (!L.wqkv_scale || !L.wo_scale || !L.wi_scale || !L.wo2_scale))
      return fail(TTE_E_INVALID, "layer " + std::to_string(l) + ": a scale / record pointer is NULL");
  }
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) {
    (void)hipGetLastError();
    return fail(TTE_E_DEVICE, "no HIP device present");
  }
  const Layout L = layout_of(c);
  if (!d_workspace) return fail(TTE_E_INVALID, "d_workspace is NULL");
  if (((uintptr_t)d_workspace & 255u) != 0) return fail(TTE_E_INVALID, "d_workspace must be 256-byte aligned");
  if (workspace_bytes < L.total) return fail(TTE_E_NOMEM, "workspace smaller than tte_workspace_size");

  tte_model* m = new (std::nothrow) tte_model();
  if (!m) return fail(TTE_E_NOMEM, "host allocation failed");
  m->cfg = c;
  m->w = *w;
  m->layers.assign(w->layers, w->layers + c.n_layers);
  m->w.layers = m->layers.data();
  m->L = L;
  m->ws = reinterpret_cast<uint8_t*>(d_workspace);
  (void)hipGetDevice(&m->device);
  uint8_t* b = m->ws;
  m->x = b + L.x;
  m->xa = b + L.xa;
  m->ascale = reinterpret_cast<float*>(b + L.ascale);
  m->qkv = b + L.qkv;
  m->vt = b + L.vt;
  m->o = b + L.o;
  m->y = b + L.y;
  m->kpart = reinterpret_cast<float*>(b + L.kpart);
  m->seg = reinterpret_cast<Seg*>(b + L.seg);
  m->d_io = reinterpret_cast<PackIO*>(b + L.off);
  m->d_off = reinterpret_cast<int*>(b + L.off + sizeof(PackIO));
  m->d_unit = m->d_off + 1;
  m->d_qunit = m->d_off + 2;
  m->partial = reinterpret_cast<float*>(b + L.partial);
  m->cosg = reinterpret_cast<const float*>(b + L.cosg);
  m->sing = reinterpret_cast<const float*>(b + L.sing);
  m->cosl = reinterpret_cast<const float*>(b + L.cosl);
  m->sinl = reinterpret_cast<const float*>(b + L.sinl);

  // RoPE tables: angle p * base^(-2c/64), rotate-half pairs (c, c + 32),
  // evaluated in double and rounded to fp32.
  const size_t n = (size_t)c.max_text_len * 32;
  std::vector<float> tab(4 * n);
  const double bases[2] = {c.rope_base_global, c.rope_base_local};
  for (int which = 0; which < 2; ++which)
    for (int p = 0; p < c.max_text_len; ++p)
      for (int k = 0; k < 32; ++k) {
        const double ang = (double)p * std::pow(bases[which], -2.0 * k / 64.0);
        tab[(2 * which) * n + (size_t)p * 32 + k] = (float)std::cos(ang);
        tab[(2 * which + 1) * n + (size_t)p * 32 + k] = (float)std::sin(ang);
      }
  tte_status st = TTE_OK;
  const size_t dst[4] = {L.cosg, L.sing, L.cosl, L.sinl};
  for (int i = 0; i < 4 && st == TTE_OK; ++i)
    st = hip_check(hipMemcpy(b + dst[i], tab.data() + i * n, n * 4, hipMemcpyHostToDevice), "hipMemcpy(rope)");
  // the slack columns of V^T are read (and multiplied by zero weights) by
  // key tiles that run past the pack: keep them finite
  if (st == TTE_OK)
    st = hip_check(hipMemset(m->vt, 0, (size_t)c.hidden * L.vt_stride * act_bytes(c.precision)), "hipMemset(vt)");
  for (int i = 0; i < L.n_guards && st == TTE_OK; ++i)
    st = hip_check(hipMemset(b + L.guard[i], GUARD_FILL, GUARD_BYTES), "hipMemset(guard)");
  if (st == TTE_OK)
    st = hip_check(hipHostMalloc((void**)&m->h_stage, sizeof(int) * stage_ints(c) * STAGE_SLOTS, hipHostMallocDefault),
                   "hipHostMalloc");
  int n_ev = 0;
  for (; st == TTE_OK && n_ev < STAGE_SLOTS; ++n_ev)
    st = hip_check(hipEventCreateWithFlags(&m->stage_ev[n_ev], hipEventDisableTiming), "hipEventCreate");
  if (st != TTE_OK) {
    for (int i = 0; i + 1 < n_ev; ++i) (void)hipEventDestroy(m->stage_ev[i]);
    if (m->h_stage) (void)hipHostFree(m->h_stage);
    delete m;
    return st;
  }
  *out = m;
  log_line("create: precision %d, %d layers, hidden %d, intermediate %d, max_tokens %d, max_texts %d, "
           "max_text_len %d, flags %d, workspace %zu bytes%s, device %d",
           c.precision, c.n_layers, c.hidden, c.intermediate, c.max_tokens, c.max_texts, c.max_text_len, c.flags,
           (size_t)L.total, L.n_guards ? " (with guards)" : "", m->device);
  return TTE_OK;
}

tte_status tte_embed(tte_model* m, const int32_t* d_token_ids, int32_t n_tokens, const int32_t* h_offsets,
                     int32_t n_texts, float* d_out, void* stream) {
  return run_pass(m, d_token_ids, n_tokens, h_offsets, n_texts, d_out, nullptr, 0, stream);
}

tte_status tte_embed_tokens(tte_model* m, const int32_t* d_token_ids, int32_t n_tokens, const int32_t* h_offsets,
                            int32_t n_texts, float* d_out_tokens, void* stream) {
  if (!d_out_tokens && n_texts > 0) return fail(TTE_E_INVALID, "d_out_tokens is NULL");
  return run_pass(m, d_token_ids, n_tokens, h_offsets, n_texts, nullptr, nullptr, 0, stream, d_out_tokens);
}

tte_status tte_similarity(const float* d_emb, int32_t n, int32_t dim, float* d_sim, void* stream) {
  if (n < 0) return fail(TTE_E_INVALID, "n must be >= 0");
  if (dim <= 0 || dim % 16 != 0) return fail(TTE_E_UNSUPPORTED, "dim must be a positive multiple of 16");
  if (n > 65536) return fail(TTE_E_UNSUPPORTED, "n above 65536");
  if (n == 0) return TTE_OK;
  if (!d_emb || !d_sim) return fail(TTE_E_INVALID, "NULL buffer");
  (void)hipGetLastError();
  launch_similarity(d_emb, n, dim, d_sim, reinterpret_cast<hipStream_t>(stream));
  return hip_check(hipGetLastError(), "kernel launch");
}

tte_status tte_embed_trace(tte_model* m, const int32_t* d_token_ids, int32_t n_tokens, const int32_t* h_offsets,
                           int32_t n_texts, float* d_out, float* d_states, int32_t n_dump, void* stream) {
  if (!d_states) return fail(TTE_E_INVALID, "d_states is NULL");
  return run_pass(m, d_token_ids, n_tokens, h_offsets, n_texts, d_out, d_states, n_dump, stream);
}

tte_status tte_destroy(tte_model* m) {
  if (!m) return fail(TTE_E_INVALID, "model is NULL");
  for (int i = 0; i < STAGE_SLOTS; ++i) {
    if (m->stage_pending[i]) (void)hipEventSynchronize(m->stage_ev[i]);
    (void)hipEventDestroy(m->stage_ev[i]);
  }
  (void)hipHostFree(m->h_stage);
  for (hipEvent_t e : m->ev) (void)hipEventDestroy(e);
  // replays may still be running on the caller's streams: each graph waits
  // for its own last replay
  tte_status st = TTE_OK;
  if (!m->graphs.empty()) (void)hipSetDevice(m->device);
  for (auto& g : m->graphs) {
    const tte_status r = release_graph(g);
    if (st == TTE_OK) st = r;
  }
  delete m;
  return st;
}

tte_status tte_op_layernorm(const float* d_x, const float* d_gamma, int32_t rows, int32_t width, float eps,
                            int32_t out_kind, void* d_out, float* d_scale, void* stream) {
  if (rows < 0) return fail(TTE_E_INVALID, "rows must be >= 0");
  if (!row_width_supported(width)) return fail(TTE_E_UNSUPPORTED, "unsupported row width");
  if (out_kind < TTE_OUT_F32 || out_kind > TTE_OUT_I8) return fail(TTE_E_INVALID, "bad out_kind");
  if (rows == 0) return TTE_OK;
  if (!d_x || !d_out || (out_kind == TTE_OUT_I8 && !d_scale)) return fail(TTE_E_INVALID, "NULL buffer");
  if (d_gamma && !(eps > 0.f)) return fail(TTE_E_INVALID, "eps must be > 0");
  (void)hipGetLastError();
  launch_ln(d_x, O_F32, d_gamma, rows, width, eps, out_kind, d_out, d_scale, reinterpret_cast<hipStream_t>(stream));
  return hip_check(hipGetLastError(), "kernel launch");
}

tte_status tte_op_quant7(const float* d_x, int32_t rows, int32_t width, int8_t* d_q, float* d_scale, void* stream) {
  if (rows < 0) return fail(TTE_E_INVALID, "rows must be >= 0");
  if (!row_width_supported(width)) return fail(TTE_E_UNSUPPORTED, "unsupported row width");
  if (rows == 0) return TTE_OK;
  if (!d_x || !d_q || !d_scale) return fail(TTE_E_INVALID, "NULL buffer");
  (void)hipGetLastError();
  launch_quant7(d_x, rows, width, d_q, d_scale, reinterpret_cast<hipStream_t>(stream));
  return hip_check(hipGetLastError(), "kernel launch");
}

tte_status tte_op_gemm(int32_t precision, int32_t epilogue, const void* d_a, const float* d_a_scale, const void* d_w,
                       const float* d_w_scale, int32_t M, int32_t N, int32_t K, void* d_c, int32_t out_kind,
                       void* stream) {
  if (precision < TTE_FP32 || precision > TTE_INT4) return fail(TTE_E_INVALID, "bad precision");
  if (epilogue < TTE_EPI_STORE || epilogue > TTE_EPI_GEGLU) return fail(TTE_E_INVALID, "bad epilogue");
  if (M < 0 || N <= 0 || K <= 0) return fail(TTE_E_INVALID, "M must be >= 0, N and K > 0");
  if (K % 128 != 0) return fail(TTE_E_UNSUPPORTED, "K must be a multiple of 128");
  if (epilogue == TTE_EPI_GEGLU ? (N % 64 != 0) : (N % 128 != 0))
    return fail(TTE_E_UNSUPPORTED, "N must be a multiple of 128 (64 for GEGLU)");
  if (out_kind != TTE_OUT_F32 && out_kind != TTE_OUT_BF16) return fail(TTE_E_INVALID, "out_kind must be F32 or BF16");
  if (epilogue == TTE_EPI_RESIDUAL && out_kind != TTE_OUT_F32 && precision != TTE_BF16)
    return fail(TTE_E_INVALID, "RESIDUAL needs fp32 C (bf16 C with TTE_BF16 only)");
  if (!weight_offsets_fit(precision, epilogue == TTE_EPI_GEGLU ? 2 * (int64_t)N : N, K))
    return fail(TTE_E_UNSUPPORTED, "W is 4 GiB or larger (the kernels address its rows with 32-bit byte offsets)");
  if (M == 0) return TTE_OK;
  if (!d_a || !d_w || !d_c) return fail(TTE_E_INVALID, "NULL buffer");
  if (precision >= TTE_INT8 && (!d_a_scale || !d_w_scale)) return fail(TTE_E_INVALID, "int8 / int4 need both scales");
  if (precision == TTE_INT4 && K % 256 != 0) return fail(TTE_E_UNSUPPORTED, "TTE_INT4 needs K a multiple of 256");
  (void)hipGetLastError();
  launch_gemm(precision, epilogue, d_a, d_a_scale, d_w, d_w_scale, M, N, K, d_c, out_kind,
              reinterpret_cast<hipStream_t>(stream));
  return hip_check(hipGetLastError(), "kernel launch");
}

tte_status tte_op_gemm_splitk(int32_t precision, const void* d_a, const float* d_a_scale, const void* d_w,
                              const float* d_w_scale, int32_t M, int32_t N, int32_t K, int32_t splits,
                              float* d_partials, void* stream) {
  if (precision < TTE_FP32 || precision > TTE_INT4) return fail(TTE_E_INVALID, "bad precision");
  if (M < 0 || N <= 0 || K <= 0 || splits < 1) return fail(TTE_E_INVALID, "M must be >= 0, N, K, splits > 0");
  const int es = precision == TTE_FP32 ? 4 : (precision == TTE_BF16 ? 2 : 1);
  if (N % 128 != 0 || K % splits != 0 || ((K / splits) * es) % 128 != 0)
    return fail(TTE_E_UNSUPPORTED, "N must be a multiple of 128 and each K part a multiple of 128 bytes");
  if (precision == TTE_INT4 && K % 256 != 0) return fail(TTE_E_UNSUPPORTED, "TTE_INT4 needs K a multiple of 256");
  if (!weight_offsets_fit(precision, N, K))
    return fail(TTE_E_UNSUPPORTED, "W is 4 GiB or larger (the kernels address its rows with 32-bit byte offsets)");
  if (M == 0) return TTE_OK;
  if (!d_a || !d_w || !d_partials || (precision >= TTE_INT8 && (!d_a_scale || !d_w_scale)))
    return fail(TTE_E_INVALID, "NULL buffer");
  (void)hipGetLastError();
  launch_gemm_splitk(precision, d_a, d_a_scale, d_w, d_w_scale, M, N, K, splits, d_partials,
                     reinterpret_cast<hipStream_t>(stream));
  return hip_check(hipGetLastError(), "kernel launch");
}

tte_status tte_op_resid_ln(float* d_x, const float* d_partials, int32_t splits, const float* d_gamma, int32_t rows,
                           int32_t width, float eps, int32_t out_kind, void* d_out, float* d_scale, void* stream) {
  if (rows < 0 || splits < 0) return fail(TTE_E_INVALID, "rows and splits must be >= 0");
  if (!row_width_supported(width)) return fail(TTE_E_UNSUPPORTED, "unsupported row width");
  if (out_kind < -1 || out_kind > TTE_OUT_I8) return fail(TTE_E_INVALID, "bad out_kind");
  if (rows == 0) return TTE_OK;
  if (!d_x || (splits > 0 && !d_partials) || (out_kind >= 0 && !d_out) || (out_kind == TTE_OUT_I8 && !d_scale))
    return fail(TTE_E_INVALID, "NULL buffer");
  if (d_gamma && !(eps > 0.f)) return fail(TTE_E_INVALID, "eps must be > 0");
  (void)hipGetLastError();
  launch_resid_ln(d_x, O_F32, d_partials, splits, d_gamma, rows, width, eps, out_kind, d_out, d_scale,
                  reinterpret_cast<hipStream_t>(stream));
  return hip_check(hipGetLastError(), "kernel launch");
}

tte_status tte_op_attention(tte_model* m, int32_t layer, const void* d_qkv, int32_t n_tokens, const int32_t* h_offsets,
                            int32_t n_texts, void* d_o, void* stream) {
  if (!m) return fail(TTE_E_INVALID, "model is NULL");
  if (layer < 0 || layer >= m->cfg.n_layers) return fail(TTE_E_INVALID, "layer out of range");
  tte_status st = check_pack(m->cfg, n_tokens, h_offsets, n_texts);
  if (st != TTE_OK) return st;
  if (n_texts == 0) return TTE_OK;
  if (!d_qkv || !d_o) return fail(TTE_E_INVALID, "NULL buffer");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  int n_units = 0;
  st = upload_pack(m, h_offsets, n_texts, &n_units, s);
  if (st != TTE_OK) return st;
  k_seg<<<(n_tokens + 255) / 256, 256, 0, s>>>(m->d_off, n_texts, n_tokens, m->seg);
  const int glob = (layer % m->cfg.global_every) == 0;
  const int prec = m->cfg.precision == TTE_BF16 ? P_BF16 : P_F32;
  const QkvOut qo{m->seg, glob ? m->cosg : m->cosl, glob ? m->sing : m->sinl, m->vt, m->L.vt_stride, m->cfg.hidden};
  launch_qkv_prep(prec, d_qkv, m->qkv, qo, n_tokens, s);
  launch_attention(prec, m->qkv, m->vt, m->L.vt_stride, d_o, m->seg, n_tokens, m->cfg.n_heads, glob, m->cfg.window,
                   n_tokens / n_texts, s, m->d_off, m->d_qunit, n_texts);
  return hip_check(hipGetLastError(), "kernel launch");
}

tte_status tte_op_qkv(tte_model* m, int32_t layer, const void* d_a, const float* d_a_scale, int32_t n_tokens,
                      const int32_t* h_offsets, int32_t n_texts, void* d_qk, void* d_vt, void* stream) {
  if (!m) return fail(TTE_E_INVALID, "model is NULL");
  if (layer < 0 || layer >= m->cfg.n_layers) return fail(TTE_E_INVALID, "layer out of range");
  tte_status st = check_pack(m->cfg, n_tokens, h_offsets, n_texts);
  if (st != TTE_OK) return st;
  if (n_texts == 0) return TTE_OK;
  if (!d_a || !d_qk || !d_vt || (m->cfg.precision >= TTE_INT8 && !d_a_scale)) return fail(TTE_E_INVALID, "NULL buffer");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  int n_units = 0;
  st = upload_pack(m, h_offsets, n_texts, &n_units, s);
  if (st != TTE_OK) return st;
  k_seg<<<(n_tokens + 255) / 256, 256, 0, s>>>(m->d_off, n_texts, n_tokens, m->seg);
  const int glob = (layer % m->cfg.global_every) == 0;
  const int H = m->cfg.hidden, P = m->cfg.precision;
  const tte_layer_weights& LW = m->layers[layer];
  const QkvOut qo{m->seg, glob ? m->cosg : m->cosl, glob ? m->sing : m->sinl, m->vt, m->L.vt_stride, H};
  launch_gemm_qkv(P, d_a, d_a_scale, LW.wqkv, LW.wqkv_scale, n_tokens, H, d_qk, P == TTE_BF16 ? O_BF16 : O_F32, qo, s);
  if (P == TTE_BF16) {
    // back to token order (the workspace copy is in the attention's column
    // order, vt_col_bf16)
    const long n = (long)H * n_tokens;
    k_vt_tokens<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(reinterpret_cast<const uint16_t*>(m->vt), m->L.vt_stride,
                                                           reinterpret_cast<uint16_t*>(d_vt), n_tokens, H);
  } else {
    st = hip_check(hipMemcpy2DAsync(d_vt, (size_t)n_tokens * 4, m->vt, (size_t)m->L.vt_stride * 4,
                                    (size_t)n_tokens * 4, (size_t)H, hipMemcpyDeviceToDevice, s),
                   "hipMemcpy2DAsync(vt)");
    if (st != TTE_OK) return st;
  }
  return hip_check(hipGetLastError(), "kernel launch");
}

tte_status tte_op_pool(tte_model* m, const float* d_x, int32_t n_tokens, const int32_t* h_offsets, int32_t n_texts,
                       float* d_out, void* stream) {
  if (!m) return fail(TTE_E_INVALID, "model is NULL");
  tte_status st = check_pack(m->cfg, n_tokens, h_offsets, n_texts);
  if (st != TTE_OK) return st;
  if (n_texts == 0) return TTE_OK;
  if (!d_x || !d_out) return fail(TTE_E_INVALID, "NULL buffer");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  int n_units = 0;
  st = upload_pack(m, h_offsets, n_texts, &n_units, s);
  if (st != TTE_OK) return st;
  launch_pool(d_x, O_F32, m->w.final_norm, m->cfg.ln_eps, m->cfg.hidden, m->d_off, m->d_unit, n_texts, n_units, m->partial,
              d_out, s);
  return hip_check(hipGetLastError(), "kernel launch");
}

tte_status tte_op_pool_static(tte_model* m, const float* d_x, int32_t n_tokens, const int32_t* h_offsets,
                              int32_t n_texts, float* d_out, void* stream) {
  if (!m) return fail(TTE_E_INVALID, "model is NULL");
  tte_status st = check_pack(m->cfg, n_tokens, h_offsets, n_texts);
  if (st != TTE_OK) return st;
  if (n_texts == 0) return TTE_OK;
  if (!d_x || !d_out) return fail(TTE_E_INVALID, "NULL buffer");
  const int H = m->cfg.hidden;
  int64_t n_units = 0;
  for (int b = 0; b < n_texts; ++b) n_units += (h_offsets[b + 1] - h_offsets[b] + POOL_ROWS - 1) / POOL_ROWS;
  // layout: offsets [n_texts + 1], unit starts [n_texts + 1], then (256-byte
  // aligned) the partial sums [n_units, H] fp32
  const size_t head = al(sizeof(int) * 2 * ((size_t)n_texts + 1));
  const size_t need = head + (size_t)n_units * H * 4;
  if (need > STATIC_SCRATCH_BYTES)
    return fail(TTE_E_UNSUPPORTED, "tte_op_pool_static: the pack needs " + std::to_string(need) +
                                       " bytes of scratch (offsets + ceil(len/32) partial rows of hidden fp32 per "
                                       "text); the static scratch holds " + std::to_string(STATIC_SCRATCH_BYTES));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  st = hip_check(hipSetDevice(m->device), "hipSetDevice");
  if (st != TTE_OK) return st;
  uint8_t* base = nullptr;
  st = scratch_on(m->device, &base);
  if (st != TTE_OK) return st;
  (void)hipGetLastError();
  int* d_off = reinterpret_cast<int*>(base);
  st = stage_offsets_to(m, h_offsets, n_texts, (int)n_units, d_off, s);
  if (st != TTE_OK) return st;
  launch_pool(d_x, O_F32, m->w.final_norm, m->cfg.ln_eps, H, d_off, d_off + (n_texts + 1), n_texts, (int)n_units,
              reinterpret_cast<float*>(base + head), d_out, s);
  return hip_check(hipGetLastError(), "kernel launch");
}

tte_status tte_profile_start(tte_model* m, uint32_t class_mask, int32_t max_launches) {
  if (!m) return fail(TTE_E_INVALID, "model is NULL");
  if (max_launches <= 0) return fail(TTE_E_INVALID, "max_launches must be positive");
  for (hipEvent_t e : m->ev) (void)hipEventDestroy(e);
  m->ev.assign(2 * (size_t)max_launches, nullptr);
  m->ev_cls.assign((size_t)max_launches, 0);
  for (auto& e : m->ev) {
    tte_status st = hip_check(hipEventCreateWithFlags(&e, hipEventDisableSystemFence), "hipEventCreate");
    if (st != TTE_OK) return st;
  }
  m->ev_used = 0;
  m->ev_overflow = false;
  m->prof_mask = class_mask;
  m->prof_on = true;
  return TTE_OK;
}

tte_status tte_graph_stats(const tte_model* m, int32_t* n_shapes, int32_t* n_graphs, int64_t* n_replays) {
  if (!m || !n_shapes || !n_graphs || !n_replays) return fail(TTE_E_INVALID, "NULL argument");
  *n_shapes = (int32_t)m->graphs.size();
  int32_t g = 0;
  for (const auto& e : m->graphs) g += e.exec != nullptr;
  *n_graphs = g;
  *n_replays = m->graph_replays;
  return TTE_OK;
}

tte_status tte_profile_stop(tte_model* m, double* ms_per_class, int64_t* launches_per_class) {
  if (!m) return fail(TTE_E_INVALID, "model is NULL");
  if (!ms_per_class || !launches_per_class) return fail(TTE_E_INVALID, "NULL output");
  m->prof_on = false;
  for (int k = 0; k < TTE_K_COUNT; ++k) {
    ms_per_class[k] = 0.0;
    launches_per_class[k] = 0;
  }
  for (int i = 0; i < m->ev_used; ++i) {
    tte_status st = hip_check(hipEventSynchronize(m->ev[2 * i + 1]), "hipEventSynchronize");
    if (st != TTE_OK) return st;
    float ms = 0.f;
    st = hip_check(hipEventElapsedTime(&ms, m->ev[2 * i], m->ev[2 * i + 1]), "hipEventElapsedTime");
    if (st != TTE_OK) return st;
    ms_per_class[m->ev_cls[i]] += ms;
    launches_per_class[m->ev_cls[i]] += 1;
  }
  for (hipEvent_t e : m->ev) (void)hipEventDestroy(e);
  m->ev.clear();
  m->ev_used = 0;
  if (m->ev_overflow) return fail(TTE_E_NOMEM, "more launches than max_launches: later ones were not timed");
  return TTE_OK;
}

}  // extern "C"
