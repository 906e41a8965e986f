// C ABI of the EAGLE draft-and-verify hot path (declared in include/eagle.h).
// Host-side argument checks, workspace carving and the launch sequence of a
// draft step; every computation runs in the HIP kernels.
#include <hip/hip_runtime.h>
#include <string.h>

#include <vector>

#include "../../include/eagle.h"
#include "gemm.h"
#include "kernels.h"

namespace {

thread_local int g_last_hip = 0;

int hip_fail(hipError_t e) {
  g_last_hip = (int)e;
  return EAGLE_EHIP;
}

// gfx950 check, cached per device.
int check_device() {
  static signed char state[64] = {0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= 64) return EAGLE_EUNSUPPORTED;
  if (state[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e);
    state[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
  }
  return state[dev] == 1 ? EAGLE_OK : EAGLE_EUNSUPPORTED;
}

bool shape_ok(const eagle_shape* s) {
  if (!s) return false;
  if (s->d <= 0 || s->n_heads <= 0 || s->n_kv_heads <= 0 || s->head_dim <= 0 || s->ffn <= 0 || s->vocab <= 0)
    return false;
  if (s->n_heads % s->n_kv_heads) return false;
  if (s->head_dim % 2) return false;
  if (!(s->rms_eps > 0.f) || !(s->rope_theta > 0.f)) return false;
  if (s->dtype != EAGLE_F32 && s->dtype != EAGLE_BF16) return false;
  return true;
}

// Supported sizes of the kernels (beyond plain validity).
int shape_supported(const eagle_shape* s) {
  if (s->vocab % 4) return EAGLE_EUNSUPPORTED;
  if (s->dtype == EAGLE_BF16) {
    if (s->head_dim != 128) return EAGLE_EUNSUPPORTED;
    if (s->d % 128 || s->ffn % 128 || (s->n_heads * s->head_dim) % 128) return EAGLE_EUNSUPPORTED;
  } else {
    if (s->head_dim != 16 && s->head_dim != 64 && s->head_dim != 128) return EAGLE_EUNSUPPORTED;
  }
  return EAGLE_OK;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Measurement hook state (see eagle_profile_enable).
struct ProfRec {
  int role;
  double bytes, flops;
};
struct Prof {
  bool on = false;
  std::vector<hipEvent_t> ev;  // 2 per launch
  std::vector<ProfRec> rec;
  size_t used = 0;
};
Prof g_prof;

// Brackets one launch; returns the launch's error.
template <typename F>
hipError_t timed(hipStream_t st, int role, double bytes, double flops, F&& launch, bool kernel_events = false) {
  const bool rec = g_prof.on && g_prof.used < g_prof.rec.size();
  // a single-kernel GEMM records its own execution start/stop; other launches
  // are bracketed by events on the stream (dispatch gap included)
  if (rec && kernel_events)
    gemm_set_kernel_events(g_prof.ev[2 * g_prof.used], g_prof.ev[2 * g_prof.used + 1]);
  else if (rec)
    hipEventRecord(g_prof.ev[2 * g_prof.used], st);
  hipError_t e = launch();
  if (rec) {
    if (kernel_events)
      gemm_set_kernel_events(nullptr, nullptr);
    else
      hipEventRecord(g_prof.ev[2 * g_prof.used + 1], st);
    g_prof.rec[g_prof.used] = ProfRec{role, bytes, flops};
    ++g_prof.used;
  }
  return e;
}

struct DraftWs {
  float* xin;  // [f_parent ; e(token)], 2d per row
  float* x;
  float* xg;  // x * gain of the next RMSNorm (first x * g1, then h * g2)
  float* sumsq1;
  float* qkv;
  void* qrot;
  float* attn_part;
  void* attn;
  float* h;
  float* sumsq2;
  void* act;
  float* gemm_part;
  void* topk;
  // split bf16 operands (hi rows, then lo rows) handed from one GEMM's epilogue
  // (or attention) to the next GEMM (bf16 weights, more than 16 rows): d wide,
  // max(ffn, hq) wide
  uint16_t* xb_d;
  uint16_t* xb_f;
  size_t total;
};

// Carves the workspace; with base == nullptr only computes the size.
DraftWs carve(const eagle_shape* s, int M, int B, int max_prefix, char* base) {
  DraftWs w{};
  const int hq = s->n_heads * s->head_dim, hkv = s->n_kv_heads * s->head_dim;
  const int nqkv = hq + 2 * hkv;
  const int npart = s->d / 16 + 2;  // >= partial tiles of any GEMM producing a d-wide output
  // most splits an attention call over at most M rows can use: the plan
  // depends on the query blocks per (sequence, kv head), so take the largest
  // over every block count a call could have (64 queries per block)
  int nsplit = 1;
  const int max_q = M * (s->n_heads / s->n_kv_heads);
  for (int q = 1;; q += 64) {
    const int n = attn_plan(s->dtype == EAGLE_BF16, max_prefix, B, s->n_kv_heads, q).n_splits;
    if (n > nsplit) nsplit = n;
    if (q >= max_q) break;
  }
  size_t gp = 0;
  if (s->dtype == EAGLE_BF16) {
    const int Ns[6] = {s->d, nqkv, s->d, 2 * s->ffn, s->d, s->vocab};
    const int Ks[6] = {2 * s->d, s->d, hq, s->d, s->ffn, s->d};
    for (int i = 0; i < 6; ++i) {
      const size_t b = gemm_bf16_partial_bytes(M, Ns[i], Ks[i]);
      if (b > gp) gp = b;
    }
  }
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += align256(bytes);
    return (void*)p;
  };
  w.xin = (float*)take((size_t)M * 2 * s->d * 4);
  w.x = (float*)take((size_t)M * s->d * 4);
  w.xg = (float*)take((size_t)M * s->d * 4);
  w.sumsq1 = (float*)take((size_t)npart * M * 4);
  w.qkv = (float*)take((size_t)M * nqkv * 4);
  w.qrot = take((size_t)M * hq * 4);
  w.attn_part = (float*)take((size_t)nsplit * M * s->n_heads * (s->head_dim + 2) * 4);
  w.attn = take((size_t)M * hq * 4);
  w.h = (float*)take((size_t)M * s->d * 4);
  w.sumsq2 = (float*)take((size_t)npart * M * 4);
  w.act = take((size_t)M * s->ffn * 4);
  w.gemm_part = (float*)take(gp);
  w.topk = take(topk_workspace_bytes(M, s->vocab));
  if (s->dtype == EAGLE_BF16 && M > 16) {
    w.xb_d = (uint16_t*)take((size_t)M * s->d * 4);
    w.xb_f = (uint16_t*)take((size_t)M * (s->ffn > hq ? s->ffn : hq) * 4);
  }
  w.total = off;
  return w;
}

GemmArgs gemm_base(int M, int N, int K) {
  GemmArgs a;
  memset(&a, 0, sizeof(a));
  a.M = M;
  a.N = N;
  a.K = K;
  a.n_seg0 = N;
  a.splits = 1;
  return a;
}

}  // namespace

extern "C" {

const char* eagle_strerror(int code) {
  switch (code) {
    case EAGLE_OK: return "ok";
    case EAGLE_EINVAL: return "invalid argument";
    case EAGLE_EUNSUPPORTED: return "unsupported shape, size or device";
    case EAGLE_EWORKSPACE: return "workspace too small";
    case EAGLE_EHIP: return "HIP error";
    default: return "unknown error";
  }
}

int eagle_last_hip_error(void) { return g_last_hip; }

size_t eagle_blocked_weight_bytes(int32_t rows, int32_t cols) {
  if (rows <= 0 || cols <= 0 || cols % 128) return 0;
  return blocked_weight_bytes(rows, cols);
}

int eagle_block_weight(const void* w, int32_t rows, int32_t cols, void* out, eagle_stream_t stream) {
  if (!w || !out || rows <= 0 || cols <= 0 || cols % 128 || ((uintptr_t)w & 15) || ((uintptr_t)out & 15))
    return EAGLE_EINVAL;
  int rc = check_device();
  if (rc) return rc;
  hipError_t e = launch_block_weight(w, rows, cols, out, (hipStream_t)stream);
  return e == hipSuccess ? EAGLE_OK : hip_fail(e);
}

size_t eagle_workspace_bytes(const eagle_shape* shape, int32_t max_rows, int32_t max_batch, int32_t max_prefix_len) {
  if (!shape_ok(shape) || max_rows <= 0 || max_batch <= 0 || max_prefix_len < 0) return 0;
  return carve(shape, max_rows, max_batch, max_prefix_len, nullptr).total;
}

int eagle_softmax_topk(int32_t n_rows, int32_t vocab, const float* logits, int32_t topk, float* lse,
                       int32_t* topk_idx, float* topk_logq, void* workspace, size_t workspace_bytes,
                       eagle_stream_t stream) {
  if (n_rows < 0 || vocab <= 0 || topk < 1 || topk > vocab) return EAGLE_EINVAL;
  if (n_rows == 0) return EAGLE_OK;
  if (!logits || !lse || !topk_idx || !topk_logq || !workspace) return EAGLE_EINVAL;
  if (topk > EAGLE_MAX_TOPK || vocab % 4) return EAGLE_EUNSUPPORTED;
  if (workspace_bytes < topk_workspace_bytes(n_rows, vocab)) return EAGLE_EWORKSPACE;
  int rc = check_device();
  if (rc) return rc;
  hipError_t e = launch_softmax_topk(n_rows, vocab, logits, topk, lse, topk_idx, topk_logq, workspace,
                                     (hipStream_t)stream);
  return e == hipSuccess ? EAGLE_OK : hip_fail(e);
}

// Fusion workspace: the [l ; m ; h] rows (fp32), per-tile sums of squares of
// the bias epilogue (unused), the GEMM's prepared operand and partials.
struct FuseWs {
  float* cat;
  float* sumsq;
  float* part;
  size_t total;
};
FuseWs carve_fuse(const eagle_shape* s, int M, char* base) {
  FuseWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += align256(bytes);
    return (void*)p;
  };
  w.cat = (float*)take((size_t)M * 3 * s->d * 4);
  w.sumsq = (float*)take((size_t)(s->d / 16 + 2) * M * 4);
  w.part = (float*)take(s->dtype == EAGLE_BF16 ? gemm_bf16_partial_bytes(M, s->d, 3 * s->d) : 0);
  w.total = off;
  return w;
}

size_t eagle_fuse_workspace_bytes(const eagle_shape* shape, int32_t max_rows) {
  if (!shape_ok(shape) || max_rows <= 0) return 0;
  return carve_fuse(shape, max_rows, nullptr).total;
}

int eagle_fuse_features(const eagle_shape* shape, const void* w_fuse, const void* b_fuse, int32_t n_rows,
                        const float* low, const float* mid, const float* high, float* g, void* workspace,
                        size_t workspace_bytes, eagle_stream_t stream) {
  if (!shape_ok(shape) || n_rows < 0) return EAGLE_EINVAL;
  if (n_rows == 0) return EAGLE_OK;
  if (!w_fuse || !low || !mid || !high || !g || !workspace) return EAGLE_EINVAL;
  int rc = shape_supported(shape);
  if (rc) return rc;
  const FuseWs ws = carve_fuse(shape, n_rows, (char*)workspace);
  if (workspace_bytes < ws.total) return EAGLE_EWORKSPACE;
  rc = check_device();
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  const int d = shape->d;
  hipError_t e = launch_concat3(low, mid, high, n_rows, d, ws.cat, st);
  if (e != hipSuccess) return hip_fail(e);
  GemmArgs a = gemm_base(n_rows, d, 3 * d);
  a.w0 = w_fuse;
  a.x = ws.cat;
  a.ldx = 3 * d;
  a.y = g;
  a.ldy = d;
  a.part = ws.part;
  int np = 0;
  int epi = EPI_STORE;
  if (b_fuse) {
    a.bias = b_fuse;
    a.sumsq_out = ws.sumsq;
    epi = EPI_BIAS_SUMSQ;
  }
  e = shape->dtype == EAGLE_BF16 ? launch_gemm_bf16(a, epi, &np, st) : launch_gemm_f32(a, epi, &np, st);
  return e == hipSuccess ? EAGLE_OK : hip_fail(e);
}

static_assert(VERIFY_NOALLOC_MAX_NODES == EAGLE_VERIFY_NOALLOC_MAX_NODES, "verify scratch limit");
static_assert(kCommitOverflow == EAGLE_COMMIT_OVERFLOW && kCommitBadPath == EAGLE_COMMIT_BAD_PATH, "commit flags");

int eagle_commit(const eagle_shape* shape, int32_t batch, int32_t n_nodes, const int32_t* path,
                 const int32_t* accept_len, const int32_t* node_slot, const void* tree_k, const void* tree_v,
                 void* prefix_k, void* prefix_v, const int64_t* prefix_off, int32_t* prefix_len,
                 const int32_t* prefix_cap, int32_t* out_flags, eagle_stream_t stream) {
  if (!shape_ok(shape) || batch < 0 || n_nodes < 1) return EAGLE_EINVAL;
  if (batch == 0) return EAGLE_OK;
  if (!path || !accept_len || !tree_k || !tree_v || !prefix_k || !prefix_v || !prefix_off || !prefix_len ||
      !out_flags)
    return EAGLE_EINVAL;
  if (n_nodes > EAGLE_MAX_SLOTS) return EAGLE_EUNSUPPORTED;
  int rc = check_device();
  if (rc) return rc;
  CommitArgs a;
  a.batch = batch;
  a.n_nodes = n_nodes;
  a.hkv = shape->n_kv_heads;
  a.hd = shape->head_dim;
  a.path = path;
  a.accept_len = accept_len;
  a.node_slot = node_slot;
  a.tree_k = tree_k;
  a.tree_v = tree_v;
  a.prefix_k = prefix_k;
  a.prefix_v = prefix_v;
  a.prefix_off = prefix_off;
  a.prefix_len = prefix_len;
  a.prefix_cap = prefix_cap;
  a.out_flags = out_flags;
  hipError_t e = launch_commit(a, shape->dtype == EAGLE_BF16, (hipStream_t)stream);
  return e == hipSuccess ? EAGLE_OK : hip_fail(e);
}

int eagle_catchup_rows(int32_t batch, int32_t n_nodes, int32_t max_depth, const int32_t* tree_token,
                       const int32_t* path, const int32_t* accept_len, const int32_t* next_token,
                       const int32_t* prefix_len, int32_t feat_row0, int32_t* row_token, int32_t* row_parent,
                       int32_t* row_pos, int32_t* row_slot, uint64_t* row_mask, int32_t* row_start, int32_t* last_row,
                       int32_t* count, eagle_stream_t stream) {
  if (batch < 0 || n_nodes < 1 || max_depth < 0 || feat_row0 < 0) return EAGLE_EINVAL;
  if (batch == 0) return EAGLE_OK;
  if (!tree_token || !path || !accept_len || !next_token || !prefix_len || !row_token || !row_parent || !row_pos ||
      !row_slot || !row_mask || !row_start || !last_row || !count)
    return EAGLE_EINVAL;
  if (n_nodes > EAGLE_MAX_SLOTS || max_depth + 1 > EAGLE_MAX_SLOTS) return EAGLE_EUNSUPPORTED;
  int rc = check_device();
  if (rc) return rc;
  CatchupArgs a;
  a.batch = batch;
  a.n_nodes = n_nodes;
  a.max_depth = max_depth;
  a.feat_row0 = feat_row0;
  a.tree_token = tree_token;
  a.path = path;
  a.accept_len = accept_len;
  a.next_token = next_token;
  a.prefix_len = prefix_len;
  a.row_token = row_token;
  a.row_parent = row_parent;
  a.row_pos = row_pos;
  a.row_slot = row_slot;
  a.row_mask = row_mask;
  a.row_start = row_start;
  a.last_row = last_row;
  a.count = count;
  hipError_t e = launch_catchup_rows(a, (hipStream_t)stream);
  return e == hipSuccess ? EAGLE_OK : hip_fail(e);
}

int eagle_commit_catchup(const eagle_shape* shape, int32_t batch, const int32_t* count, const void* tree_k,
                         const void* tree_v, void* prefix_k, void* prefix_v, const int64_t* prefix_off,
                         int32_t* prefix_len, const int32_t* prefix_cap, const float* feat, const int32_t* last_row,
                         float* root_feat, int32_t* out_flags, eagle_stream_t stream) {
  if (!shape_ok(shape) || batch < 0) return EAGLE_EINVAL;
  if (batch == 0) return EAGLE_OK;
  if (!count || !tree_k || !tree_v || !prefix_k || !prefix_v || !prefix_off || !prefix_len || !out_flags)
    return EAGLE_EINVAL;
  if ((feat != nullptr) != (last_row != nullptr) || (feat != nullptr) != (root_feat != nullptr)) return EAGLE_EINVAL;
  int rc = check_device();
  if (rc) return rc;
  CommitArgs a;
  memset(&a, 0, sizeof(a));
  a.batch = batch;
  a.n_nodes = EAGLE_MAX_SLOTS;
  a.hkv = shape->n_kv_heads;
  a.hd = shape->head_dim;
  a.path = nullptr;  // slot mode: slots 0..count[b]-1
  a.accept_len = count;
  a.tree_k = tree_k;
  a.tree_v = tree_v;
  a.prefix_k = prefix_k;
  a.prefix_v = prefix_v;
  a.prefix_off = prefix_off;
  a.prefix_len = prefix_len;
  a.prefix_cap = prefix_cap;
  a.out_flags = out_flags;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = launch_commit(a, shape->dtype == EAGLE_BF16, st);
  if (e != hipSuccess) return hip_fail(e);
  if (feat) {
    e = launch_gather_rows(feat, last_row, batch, shape->d, root_feat, st);
    if (e != hipSuccess) return hip_fail(e);
  }
  return EAGLE_OK;
}

int eagle_sample_topk(int32_t n_rows, int32_t vocab, const float* logits, int32_t topk, uint64_t seed, uint64_t round,
                      int32_t row_base, float* lse, int32_t* topk_idx, float* topk_logq, void* workspace,
                      size_t workspace_bytes, eagle_stream_t stream) {
  if (n_rows < 0 || vocab <= 0 || topk < 1 || topk > vocab) return EAGLE_EINVAL;
  if (n_rows == 0) return EAGLE_OK;
  if (!logits || !lse || !topk_idx || !topk_logq || !workspace) return EAGLE_EINVAL;
  if (topk > EAGLE_MAX_TOPK || vocab % 4 || vocab > TOPK_SAMPLE_MAX_VOCAB) return EAGLE_EUNSUPPORTED;
  if (workspace_bytes < topk_workspace_bytes(n_rows, vocab)) return EAGLE_EWORKSPACE;
  int rc = check_device();
  if (rc) return rc;
  const TopkSample smp{seed, round, row_base};
  hipError_t e = launch_softmax_topk(n_rows, vocab, logits, topk, lse, topk_idx, topk_logq, workspace,
                                     (hipStream_t)stream, &smp);
  return e == hipSuccess ? EAGLE_OK : hip_fail(e);
}

int eagle_draft_step(const eagle_shape* shape, const eagle_weights* w, int32_t flags, const eagle_rows* rows,
                     const float* feat_in, const eagle_kv* kv, const eagle_draft_out* out, void* workspace,
                     size_t workspace_bytes, eagle_stream_t stream) {
  if (!shape_ok(shape) || !w || !rows || !out) return EAGLE_EINVAL;
  if (flags & ~(EAGLE_HEAD_ONLY | EAGLE_ACT_BF16 | EAGLE_SAMPLE_CHILDREN | EAGLE_FEATURES_ONLY)) return EAGLE_EINVAL;
  if ((flags & EAGLE_HEAD_ONLY) && (flags & EAGLE_FEATURES_ONLY)) return EAGLE_EINVAL;
  const bool sample = flags & EAGLE_SAMPLE_CHILDREN;
  const bool feat_only = flags & EAGLE_FEATURES_ONLY;
  if (sample && shape && shape->vocab > TOPK_SAMPLE_MAX_VOCAB) return EAGLE_EUNSUPPORTED;
  const bool head_only = flags & EAGLE_HEAD_ONLY;
  const int act16 = (flags & EAGLE_ACT_BF16) ? 1 : 0;
  if (act16 && shape && shape->dtype != EAGLE_BF16) return EAGLE_EINVAL;  // a bf16 rounding of an fp32 workload
  const int M = rows->n_rows;
  if (M < 0 || rows->batch <= 0) return EAGLE_EINVAL;
  if (M == 0) return EAGLE_OK;
  if (!feat_in || !rows->parent || !workspace) return EAGLE_EINVAL;
  if (!feat_only) {
    if (!out->logits || !out->lse || !out->topk_idx || !out->topk_logq || !w->lm_head) return EAGLE_EINVAL;
    if (out->topk < 1 || out->topk > shape->vocab) return EAGLE_EINVAL;
    if (out->topk > EAGLE_MAX_TOPK) return EAGLE_EUNSUPPORTED;
  }
  int rc = shape_supported(shape);
  if (rc) return rc;
  const eagle_shape& s = *shape;
  const bool bf16 = s.dtype == EAGLE_BF16;
  if (!head_only) {
    if (!kv || !out->feat || !rows->row_start || !rows->token || !rows->pos || !rows->slot || !rows->mask)
      return EAGLE_EINVAL;
    if (!w->embed || !w->fc_w || !w->fc_b || !w->norm1 || !w->norm2 || !w->wq || !w->wk || !w->wv || !w->wo ||
        !w->w_gate || !w->w_up || !w->w_down)
      return EAGLE_EINVAL;
    if (!kv->prefix_len || !kv->tree_k || !kv->tree_v || kv->max_prefix_len < 0) return EAGLE_EINVAL;
    if (kv->max_prefix_len > 0 && (!kv->prefix_k || !kv->prefix_v || !kv->prefix_off)) return EAGLE_EINVAL;
    if (rows->max_rows_per_seq <= 0 || rows->max_rows_per_seq > M) return EAGLE_EINVAL;
  }
  const int maxL = head_only ? 0 : kv->max_prefix_len;
  DraftWs ws = carve(shape, M, rows->batch, maxL, (char*)workspace);
  if (workspace_bytes < ws.total) return EAGLE_EWORKSPACE;
  rc = check_device();
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  const double wbytes = bf16 ? 2.0 : 4.0;
  // algorithmic bytes of a GEMM launch: weights once, fp32 activations in and out
  auto gemm = [&](GemmArgs a, int epi, int* np, int role) -> hipError_t {
    int dummy = 0;
    a.part = ws.gemm_part;  // split-K partials of the tiled kernel (+ the bf16 operand)
    a.act_bf16 = act16;
    const int nout = (epi == EPI_SWIGLU) ? a.ffn : a.N;
    const double out_bytes = (epi == EPI_ROPE) ? 4.0 * a.M * a.rp_hq * a.rp_hd + 2.0 * wbytes * a.M * a.rp_hkv * a.rp_hd
                                               : 4.0 * a.M * nout;
    // (the normalised copy of a SUMSQ epilogue counts once, whether written as y2 or handed over)
    const bool normed = a.y2 || (a.gain_out && a.xb_out);
    const double bytes = wbytes * a.N * a.K + 4.0 * a.M * a.K + out_bytes + (normed ? 4.0 * a.M * a.N : 0.0);
    const double flops = 2.0 * a.M * a.N * a.K;
    return timed(
        st, role, bytes, flops,
        [&] {
          return bf16 ? launch_gemm_bf16(a, epi, np ? np : &dummy, st)
                      : launch_gemm_f32(a, epi, np ? np : &dummy, st);
        },
        bf16 && a.M <= 16);
  };
  hipError_t e;
  const int d = s.d, hq = s.n_heads * s.head_dim, hkv = s.n_kv_heads * s.head_dim, F = s.ffn;
  // the skinny QKV GEMM rotates q, k and writes the tree slots in its epilogue up to
  // M = 8 (one 16-row weight tile per workgroup); above, the four-tile QKV variant
  // plus the RoPE launch is faster (measured on the 7B shapes)
  const bool rope_fused = bf16 && M <= 8 && s.head_dim % 16 == 0;
  // above 16 rows with split bf16 operands, each GEMM takes its operand from
  // the producer's epilogue (the previous GEMM's, or attention's), unscaled, and
  // applies the RMSNorm row scale in its own epilogue: no operand prep pass, and
  // the fp32 copies only a GEMM would read (x * g, attention out, SwiGLU out)
  // are not written
  const bool handover = bf16 && M > 16 && !act16;

  if (!head_only) {
    // a1: the rows' inputs [f_parent ; e(token)]: gathered by the FC GEMM itself
    // (its loader, or its operand prep pass) for bf16 weights, else concatenated here
    const bool gather = bf16;
    if (!gather) {
      RowSetupArgs r;
      r.n_rows = M;
      r.parent = rows->parent;
      r.token = rows->token;
      r.feat = feat_in;
      r.embed = w->embed;
      r.d = d;
      r.xin = ws.xin;
      // bytes: the gathered feature and embedding rows in, the concatenation out
      e = timed(st, EAGLE_ROLE_ROWS, 4.0 * M * d + wbytes * M * d + 8.0 * M * d, 0.0,
                [&] { return launch_row_setup(r, bf16, st); });
      if (e != hipSuccess) return hip_fail(e);
    }
    // a2: FC (+bias) = x; sums of squares and x * g1 for RMSNorm 1
    int np1 = 0, np2 = 0;
    {
      GemmArgs a = gemm_base(M, d, 2 * d);
      a.w0 = w->fc_w;
      if (bf16) a.wb0 = w->fc_w_b;
      if (gather) {
        a.gfeat = feat_in;
        a.gparent = rows->parent;
        a.gtoken = rows->token;
        a.gembed = w->embed;
        a.gd = d;
      } else {
        a.x = ws.xin;
        a.ldx = 2 * d;
      }
      a.bias = w->fc_b;
      a.y = ws.x;
      a.ldy = d;
      a.sumsq_out = ws.sumsq1;
      a.gain_out = w->norm1;
      a.y2 = handover ? nullptr : ws.xg;
      if (handover) a.xb_out = ws.xb_d;
      e = gemm(a, EPI_BIAS_SUMSQ, &np1, EAGLE_ROLE_FC);
      if (e != hipSuccess) return hip_fail(e);
    }
    // queries per (sequence, kv head) at most
    const int max_q = rows->max_rows_per_seq * (s.n_heads / s.n_kv_heads);
    // a3: RMSNorm -> [q; k; v]: (x * g1) [wq; wk; wv]^T, row scale in the epilogue
    {
      GemmArgs a = gemm_base(M, hq + 2 * hkv, d);
      a.w0 = w->wq;
      a.n_seg0 = hq;
      a.w1 = w->wk;
      a.n_seg1 = hkv;
      a.w2 = w->wv;
      if (bf16 && w->wq_b && w->wk_b && w->wv_b) {
        a.wb0 = w->wq_b;
        a.wb1 = w->wk_b;
        a.wb2 = w->wv_b;
      }
      a.x = ws.xg;
      a.ldx = d;
      a.sumsq_in = ws.sumsq1;
      a.n_part_in = np1;
      a.eps = s.rms_eps;
      if (handover) a.xb_in = ws.xb_d;
      if (rope_fused) {  // a4 in the epilogue: rotated q out, k and v into the rows' tree slots
        a.y = (float*)ws.qrot;
        a.ldy = hq;
        a.rp_pos = rows->pos;
        a.rp_slot = rows->slot;
        a.rp_row_start = rows->row_start;
        a.rp_batch = rows->batch;
        a.rp_tree_k = kv->tree_k;
        a.rp_tree_v = kv->tree_v;
        a.rp_hd = s.head_dim;
        a.rp_hq = s.n_heads;
        a.rp_hkv = s.n_kv_heads;
        a.rp_theta = s.rope_theta;
        e = gemm(a, EPI_ROPE, nullptr, EAGLE_ROLE_QKV);
      } else {
        a.y = ws.qkv;
        a.ldy = hq + 2 * hkv;
        e = gemm(a, EPI_STORE, nullptr, EAGLE_ROLE_QKV);
      }
      if (e != hipSuccess) return hip_fail(e);
    }
    // a4: RoPE at each row's position; k, v into the rows' tree slots
    if (!rope_fused) {
      RopeArgs r;
      r.qkv = ws.qkv;
      r.pos = rows->pos;
      r.slot = rows->slot;
      r.row_start = rows->row_start;
      r.batch = rows->batch;
      r.q_out = (float*)ws.qrot;
      r.tree_k = kv->tree_k;
      r.tree_v = kv->tree_v;
      r.n_rows = M;
      r.hq = s.n_heads;
      r.hkv = s.n_kv_heads;
      r.hd = s.head_dim;
      r.theta = s.rope_theta;
      e = timed(st, EAGLE_ROLE_ROPE, 4.0 * M * (hq + 2 * hkv) + 4.0 * M * hq + 2.0 * wbytes * M * hkv, 0.0,
                [&] { return launch_rope_kv(r, bf16, st); });
      if (e != hipSuccess) return hip_fail(e);
    }
    // a5: tree attention
    {
      AttnArgs at{};
      at.q = (const float*)ws.qrot;
      at.mask = rows->mask;
      at.row_start = rows->row_start;
      at.prefix_k = kv->prefix_k;
      at.prefix_v = kv->prefix_v;
      at.prefix_off = kv->prefix_off;
      at.prefix_len = kv->prefix_len;
      at.prefix_cap = kv->prefix_cap;
      at.tree_k = kv->tree_k;
      at.tree_v = kv->tree_v;
      at.part = ws.attn_part;
      at.out = (float*)ws.attn;
      at.outb = handover ? ws.xb_f : nullptr;
      at.n_rows = M;
      at.batch = rows->batch;
      at.hq = s.n_heads;
      at.hkv = s.n_kv_heads;
      const AttnPlan plan = attn_plan(bf16, maxL, rows->batch, s.n_kv_heads, max_q);
      at.split_len = plan.split_len;
      at.n_splits = plan.n_splits;
      // bytes: each sequence's prefix K and V once (sum of the lengths when the caller gives it), q in,
      // output out; flops 4*hd per (query, key)
      const double sum_len =
          kv->prefix_len_sum > 0 ? (double)kv->prefix_len_sum : (double)kv->max_prefix_len * rows->batch;
      const double kv_bytes = 2.0 * wbytes * s.n_kv_heads * s.head_dim * sum_len;
      e = timed(st, EAGLE_ROLE_ATTN, kv_bytes + 8.0 * M * hq, 4.0 * M * s.n_heads * s.head_dim * sum_len / rows->batch,
                [&] { return launch_attention(at, bf16, s.head_dim, max_q, st); });
      if (e != hipSuccess) return hip_fail(e);
    }
    // a6: h = x + attn wo^T; sums of squares and h * g2 for RMSNorm 2
    {
      GemmArgs a = gemm_base(M, d, hq);
      a.w0 = w->wo;
      if (bf16) a.wb0 = w->wo_b;
      a.x = (const float*)ws.attn;
      a.ldx = hq;
      a.resid = ws.x;
      a.ldr = d;
      a.y = ws.h;
      a.ldy = d;
      a.sumsq_out = ws.sumsq2;
      a.gain_out = w->norm2;
      a.y2 = handover ? nullptr : ws.xg;
      if (handover) {
        a.xb_in = ws.xb_f;
        a.xb_out = ws.xb_d;
      }
      e = gemm(a, EPI_RESID_SUMSQ, &np2, EAGLE_ROLE_O);
      if (e != hipSuccess) return hip_fail(e);
    }
    // a7: RMSNorm -> SwiGLU: (h * g2) [w_gate; w_up]^T, row scale in the epilogue
    {
      GemmArgs a = gemm_base(M, 2 * F, d);
      a.w0 = w->w_gate;
      a.n_seg0 = F;
      a.w1 = w->w_up;
      a.n_seg1 = F;
      if (bf16 && w->w_gate_b && w->w_up_b) {
        a.wb0 = w->w_gate_b;
        a.wb1 = w->w_up_b;
      }
      a.ffn = F;
      a.x = ws.xg;
      a.ldx = d;
      a.sumsq_in = ws.sumsq2;
      a.n_part_in = np2;
      a.eps = s.rms_eps;
      a.yb = handover ? nullptr : (float*)ws.act;
      a.ldyb = F;
      a.part = ws.gemm_part;
      if (handover) {
        a.xb_in = ws.xb_d;
        a.xb_out = ws.xb_f;
      }
      e = gemm(a, EPI_SWIGLU, nullptr, EAGLE_ROLE_GATE_UP);
      if (e != hipSuccess) return hip_fail(e);
    }
    // f^ = h + act w_down^T
    {
      GemmArgs a = gemm_base(M, d, F);
      a.w0 = w->w_down;
      if (bf16) a.wb0 = w->w_down_b;
      a.x = (const float*)ws.act;
      a.ldx = F;
      a.resid = ws.h;
      a.ldr = d;
      a.y = out->feat;
      a.ldy = d;
      a.part = ws.gemm_part;
      if (handover) {
        a.xb_in = ws.xb_f;
        if (!feat_only) a.xb_out = ws.xb_d;
      }
      e = gemm(a, EPI_RESID, nullptr, EAGLE_ROLE_DOWN);
      if (e != hipSuccess) return hip_fail(e);
    }
  }
  if (feat_only) return EAGLE_OK;  // f^ (and the rows' k, v) are all the caller asked for
  // a8 (a0 with HEAD_ONLY): logits = f lm_head^T
  {
    GemmArgs a = gemm_base(M, s.vocab, d);
    a.w0 = w->lm_head;
    if (bf16) a.wb0 = w->lm_head_b;
    a.x = head_only ? feat_in : out->feat;
    a.xrows = head_only ? rows->parent : nullptr;
    a.ldx = d;
    a.y = out->logits;
    a.ldy = s.vocab;
    a.part = ws.gemm_part;
    if (handover && !head_only) a.xb_in = ws.xb_d;
    e = gemm(a, EPI_STORE, nullptr, EAGLE_ROLE_LM_HEAD);
    if (e != hipSuccess) return hip_fail(e);
  }
  // a9: softmax normaliser + top-k (or k sampled children)
  const TopkSample smp{out->seed, out->round, out->row_base};
  e = timed(st, EAGLE_ROLE_TOPK, 4.0 * M * s.vocab, 0.0, [&] {
    return launch_softmax_topk(M, s.vocab, out->logits, out->topk, out->lse, out->topk_idx, out->topk_logq, ws.topk,
                               st, sample ? &smp : nullptr);
  });
  if (e != hipSuccess) return hip_fail(e);
  return EAGLE_OK;
}

int eagle_profile_enable(int32_t max_launches) {
  if (max_launches <= 0) return EAGLE_EINVAL;
  eagle_profile_disable();
  g_prof.ev.resize(2 * (size_t)max_launches);
  for (auto& e : g_prof.ev) {
    hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) return hip_fail(r);
  }
  g_prof.rec.assign(max_launches, ProfRec{0, 0.0, 0.0});
  g_prof.used = 0;
  g_prof.on = true;
  return EAGLE_OK;
}

int eagle_profile_reset(void) {
  g_prof.used = 0;
  return EAGLE_OK;
}

int eagle_profile_disable(void) {
  for (auto& e : g_prof.ev)
    if (e) hipEventDestroy(e);
  g_prof.ev.clear();
  g_prof.rec.clear();
  g_prof.used = 0;
  g_prof.on = false;
  return EAGLE_OK;
}

int eagle_profile_read(int32_t role, int32_t* launches, double* total_ms, double* bytes, double* flops) {
  if (role < 0 || role >= EAGLE_ROLE_COUNT || !launches || !total_ms || !bytes || !flops) return EAGLE_EINVAL;
  int n = 0;
  double ms = 0.0, by = 0.0, fl = 0.0;
  for (size_t i = 0; i < g_prof.used; ++i) {
    if (g_prof.rec[i].role != role) continue;
    hipError_t r = hipEventSynchronize(g_prof.ev[2 * i + 1]);
    if (r != hipSuccess) return hip_fail(r);
    float t = 0.f;
    r = hipEventElapsedTime(&t, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]);
    if (r != hipSuccess) return hip_fail(r);
    ++n;
    ms += t;
    by += g_prof.rec[i].bytes;
    fl += g_prof.rec[i].flops;
  }
  *launches = n;
  *total_ms = ms;
  *bytes = by;
  *flops = fl;
  return EAGLE_OK;
}

int eagle_tree_init(int32_t batch, const eagle_pool* pool, const int32_t* root_token, int32_t root_feat_row0,
                    eagle_stream_t stream) {
  if (batch <= 0 || !pool || !root_token || root_feat_row0 < 0) return EAGLE_EINVAL;
  if (pool->cap < 1 || !pool->parent || !pool->token || !pool->depth || !pool->logv || !pool->feat_row ||
      !pool->slot || !pool->mask || !pool->count || !pool->frontier)
    return EAGLE_EINVAL;
  int rc = check_device();
  if (rc) return rc;
  PoolArgs p{pool->cap, pool->parent, pool->token, pool->depth, pool->logv, pool->feat_row, pool->slot, pool->mask,
             pool->count, pool->frontier};
  hipError_t e = launch_tree_init(batch, p, root_token, root_feat_row0, (hipStream_t)stream);
  return e == hipSuccess ? EAGLE_OK : hip_fail(e);
}

int eagle_tree_expand(int32_t batch, int32_t k, int32_t step, const int32_t* static_nchild, const eagle_pool* pool,
                      int32_t n_prev, int32_t topk, const int32_t* topk_idx, const float* topk_logq, int32_t n_next,
                      int32_t feat_row0, const int32_t* prefix_len, int32_t* next_token, int32_t* next_parent,
                      int32_t* next_pos, int32_t* next_slot, uint64_t* next_mask, int32_t* next_row_start,
                      eagle_stream_t stream) {
  if (batch <= 0 || !pool || k < 1 || step < 0 || n_prev < 1 || n_prev > EAGLE_MAX_SLOTS || n_next < 0 ||
      n_next > EAGLE_MAX_SLOTS || topk < 1 || feat_row0 < 0)
    return EAGLE_EINVAL;
  if (!topk_idx || !topk_logq || !prefix_len || !next_token || !next_parent || !next_pos || !next_slot ||
      !next_mask || !next_row_start)
    return EAGLE_EINVAL;
  if (pool->cap < 1 || !pool->parent || !pool->count || !pool->frontier) return EAGLE_EINVAL;
  if (k > topk || topk > EAGLE_MAX_TOPK) return EAGLE_EUNSUPPORTED;
  if (!static_nchild) {
    if (n_next != k && n_next != 0) return EAGLE_EINVAL;  // 0: last expansion, no next draft step
    if ((step + 1) * k > EAGLE_MAX_SLOTS) return EAGLE_EUNSUPPORTED;  // slots step*k + f < 64
    if (n_prev * k > 256) return EAGLE_EUNSUPPORTED;
  } else {
    if (pool->cap > EAGLE_MAX_SLOTS) return EAGLE_EUNSUPPORTED;  // static slot = pool id < 64
  }
  int rc = check_device();
  if (rc) return rc;
  ExpandArgs a;
  a.pool = PoolArgs{pool->cap, pool->parent, pool->token, pool->depth, pool->logv, pool->feat_row, pool->slot,
                    pool->mask, pool->count, pool->frontier};
  a.k = k;
  a.step = step;
  a.n_prev = n_prev;
  a.topk = topk;
  a.n_next = n_next;
  a.feat_row0 = feat_row0;
  a.nchild = static_nchild;
  a.topk_idx = topk_idx;
  a.topk_logq = topk_logq;
  a.prefix_len = prefix_len;
  a.next_token = next_token;
  a.next_parent = next_parent;
  a.next_pos = next_pos;
  a.next_slot = next_slot;
  a.next_row_start = next_row_start;
  a.next_mask = next_mask;
  a.batch = batch;
  hipError_t e = launch_tree_expand(a, (hipStream_t)stream);
  return e == hipSuccess ? EAGLE_OK : hip_fail(e);
}

int eagle_tree_finalize(int32_t batch, int32_t m, int32_t n_nodes, const eagle_pool* pool, const int32_t* prefix_len,
                        int32_t* tree_parent, int32_t* tree_token, int32_t* tree_depth, int32_t* tree_pool,
                        uint64_t* tree_mask, int32_t* tree_qrow, int32_t* row_token, int32_t* row_parent,
                        int32_t* row_pos, int32_t* row_slot, uint64_t* row_mask, int32_t* row_start,
                        eagle_stream_t stream) {
  if (batch <= 0 || !pool || m < 0 || n_nodes < 1 || !prefix_len) return EAGLE_EINVAL;
  if (!tree_parent || !tree_token || !tree_depth || !tree_pool || !tree_mask || !tree_qrow || !row_token ||
      !row_parent || !row_pos || !row_slot || !row_mask || !row_start)
    return EAGLE_EINVAL;
  if (n_nodes > EAGLE_MAX_SLOTS) return EAGLE_EUNSUPPORTED;
  if (pool->cap < 1 || pool->cap > 2048) return EAGLE_EUNSUPPORTED;
  // every kept node must fit: m drafted nodes and the root, or the whole pool when m = 0
  if ((m > 0 ? m + 1 : pool->cap) > n_nodes) return EAGLE_EINVAL;
  int rc = check_device();
  if (rc) return rc;
  FinalizeArgs a;
  a.pool = PoolArgs{pool->cap, pool->parent, pool->token, pool->depth, pool->logv, pool->feat_row, pool->slot,
                    pool->mask, pool->count, pool->frontier};
  a.m = m;
  a.n_nodes = n_nodes;
  a.batch = batch;
  a.prefix_len = prefix_len;
  a.tree_parent = tree_parent;
  a.tree_token = tree_token;
  a.tree_depth = tree_depth;
  a.tree_pool = tree_pool;
  a.tree_qrow = tree_qrow;
  a.tree_mask = tree_mask;
  a.row_token = row_token;
  a.row_parent = row_parent;
  a.row_pos = row_pos;
  a.row_slot = row_slot;
  a.row_start = row_start;
  a.row_mask = row_mask;
  hipError_t e = launch_tree_finalize(a, (hipStream_t)stream);
  return e == hipSuccess ? EAGLE_OK : hip_fail(e);
}

// Argument checks shared by eagle_verify and eagle_verify_noalloc.
static int verify_args_ok(int32_t batch, int32_t n_nodes, int32_t vocab, const int32_t* tree_parent,
                          const int32_t* tree_token, const float* target_logits, const float* draft_logits,
                          const int32_t* draft_row, int32_t flags, int32_t* out_path, int32_t* out_accept_len,
                          int32_t* out_next_token, int32_t* out_flags) {
  if (batch < 0 || n_nodes < 1 || vocab < 1) return EAGLE_EINVAL;
  if (batch == 0) return EAGLE_OK;
  if (!tree_parent || !tree_token || !target_logits || !draft_logits || !draft_row || !out_path ||
      !out_accept_len || !out_next_token || !out_flags)
    return EAGLE_EINVAL;
  if (flags & ~(EAGLE_VERIFY_GREEDY | EAGLE_VERIFY_IID)) return EAGLE_EINVAL;
  if (n_nodes > EAGLE_MAX_SLOTS || vocab > 32768) return EAGLE_EUNSUPPORTED;
  return EAGLE_OK;
}

static int verify_launch(int32_t batch, int32_t n_nodes, int32_t vocab, const int32_t* tree_parent,
                         const int32_t* tree_token, const float* target_logits, const float* draft_logits,
                         const int32_t* draft_row, uint64_t seed, uint64_t round, int32_t flags, int32_t* out_path,
                         int32_t* out_accept_len, int32_t* out_next_token, int32_t* out_flags, void* workspace,
                         eagle_stream_t stream) {
  VerifyArgs a;
  a.batch = batch;
  a.n_nodes = n_nodes;
  a.vocab = vocab;
  a.parent = tree_parent;
  a.token = tree_token;
  a.target = target_logits;
  a.draft = draft_logits;
  a.draft_row = draft_row;
  a.seed = seed;
  a.round = round;
  a.flags = flags;
  a.path = out_path;
  a.accept_len = out_accept_len;
  a.next_token = out_next_token;
  a.out_flags = out_flags;
  hipError_t e = launch_verify(a, workspace, (hipStream_t)stream);
  return e == hipSuccess ? EAGLE_OK : hip_fail(e);
}

int eagle_verify(int32_t batch, int32_t n_nodes, int32_t vocab, const int32_t* tree_parent, const int32_t* tree_token,
                 const float* target_logits, const float* draft_logits, const int32_t* draft_row, uint64_t seed,
                 uint64_t round, int32_t flags, int32_t* out_path, int32_t* out_accept_len, int32_t* out_next_token,
                 int32_t* out_flags, void* workspace, size_t workspace_bytes, eagle_stream_t stream) {
  int rc = verify_args_ok(batch, n_nodes, vocab, tree_parent, tree_token, target_logits, draft_logits, draft_row, flags,
                          out_path, out_accept_len, out_next_token, out_flags);
  if (rc || batch == 0) return rc;
  if (workspace && workspace_bytes < verify_workspace_bytes(batch, n_nodes)) return EAGLE_EWORKSPACE;
  rc = check_device();
  if (rc) return rc;
  return verify_launch(batch, n_nodes, vocab, tree_parent, tree_token, target_logits, draft_logits, draft_row, seed,
                       round, flags, out_path, out_accept_len, out_next_token, out_flags, workspace, stream);
}

int eagle_verify_noalloc(int32_t batch, int32_t n_nodes, int32_t vocab, const int32_t* tree_parent,
                         const int32_t* tree_token, const float* target_logits, const float* draft_logits,
                         const int32_t* draft_row, uint64_t seed, uint64_t round, int32_t flags, int32_t* out_path,
                         int32_t* out_accept_len, int32_t* out_next_token, int32_t* out_flags, eagle_stream_t stream) {
  int rc = verify_args_ok(batch, n_nodes, vocab, tree_parent, tree_token, target_logits, draft_logits, draft_row, flags,
                          out_path, out_accept_len, out_next_token, out_flags);
  if (rc || batch == 0) return rc;
  if ((int64_t)batch * n_nodes > VERIFY_NOALLOC_MAX_NODES) return EAGLE_EUNSUPPORTED;
  rc = check_device();
  if (rc) return rc;
  void* scratch = nullptr;  // the library's own per-device array, never an allocation
  hipError_t e = verify_scratch_address(&scratch);
  if (e != hipSuccess) return hip_fail(e);
  return verify_launch(batch, n_nodes, vocab, tree_parent, tree_token, target_logits, draft_logits, draft_row, seed,
                       round, flags, out_path, out_accept_len, out_next_token, out_flags, scratch, stream);
}

size_t eagle_verify_workspace_bytes(int32_t batch, int32_t n_nodes) {
  if (batch < 0 || n_nodes < 1 || n_nodes > EAGLE_MAX_SLOTS) return 0;
  return verify_workspace_bytes(batch, n_nodes);
}

}  // extern "C"
