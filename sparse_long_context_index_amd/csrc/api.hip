// C ABI of libcsa: argument validation, workspace carving and stage
// sequencing.  Every check here runs on the host before any launch; nothing
// in this file allocates, frees or synchronises.
#include <math.h>

#include <mutex>

#include "csa_common.h"

using namespace csa;

namespace {

constexpr int kAbiVersion = 3;  // 2: E4M3 indexer entry points and step fields; 3: one_sequence
constexpr int kMaxTopk = 2048;
constexpr int kMaxGridY = 65535;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }
inline bool head_dim_ok(int d) { return d == 64 || d == 128 || d == 256 || d == 512; }

csa_status hip_status(hipError_t e) { return e == hipSuccess ? CSA_OK : CSA_EHIP; }

// Workspace of the allocation-free decode step: one array in each GPU's
// memory, created when the library's code object is loaded on that GPU and
// held until the process ends.  Host code reaches it only through the device
// address hipGetSymbolAddress gives on each device (the array's name is a
// host-side stand-in, not a device address).
static __device__ __align__(256) unsigned char scratch[CSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// The scratch array's address on the current device, looked up once per
// device with that device current.
csa_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CSA_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return CSA_EHIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return CSA_OK;
}

csa_status check_index(const uint16_t* q_idx, const float* w, const uint16_t* k_idx,
                       int64_t k_rows, const int64_t* pos, const int64_t* seq_kv,
                       const int32_t* n_comp, int T, int n_ih, int ihd, int ratio,
                       const float* scores, int64_t ld) {
  if (T < 0 || n_ih < 1 || ratio < 1 || ld < 1 || k_rows < 0) return CSA_EINVAL;
  if (!q_idx || !w || !k_idx || !pos || !seq_kv || !n_comp || !scores) return CSA_EINVAL;
  if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned4(w) || !aligned4(scores))
    return CSA_EINVAL;
  if (ihd != 32 && ihd != 64 && ihd != 128) return CSA_EUNSUPPORTED;
  if (n_ih > 128 || T > kMaxGridY || ld > INT32_MAX) return CSA_EUNSUPPORTED;
  return CSA_OK;
}

csa_status check_topk(const float* scores, int64_t ld, const int64_t* pos,
                      const int32_t* n_comp, int T, int ratio, int top_k, const int32_t* idx,
                      const int32_t* count) {
  if (T < 0 || ld < 1 || ratio < 1 || top_k < 1) return CSA_EINVAL;
  if (!scores || !pos || !n_comp || !idx || !count) return CSA_EINVAL;
  if (!aligned16(scores)) return CSA_EINVAL;
  if (top_k > kMaxTopk || T > kMaxGridY || ld > INT32_MAX) return CSA_EUNSUPPORTED;
  return CSA_OK;
}

csa_status check_gather(const uint16_t* comp_kv, int64_t comp_rows, const int64_t* seq_kv,
                        const int32_t* idx, const int32_t* count, int top_k,
                        const uint16_t* swa, int64_t swa_rows, const int64_t* swa_row0,
                        const int32_t* swa_len, int window, int T, int head_dim,
                        const uint16_t* all_kv, const int32_t* n_kv) {
  if (T < 0 || top_k < 0 || window < 0 || comp_rows < 0 || swa_rows < 0) return CSA_EINVAL;
  if (!comp_kv || !seq_kv || !idx || !count || !swa || !swa_row0 || !swa_len || !all_kv || !n_kv)
    return CSA_EINVAL;
  if (!aligned16(comp_kv) || !aligned16(swa) || !aligned16(all_kv)) return CSA_EINVAL;
  if (!head_dim_ok(head_dim)) return CSA_EUNSUPPORTED;
  if (T > kMaxGridY || top_k > kMaxTopk || window > 1024) return CSA_EUNSUPPORTED;
  return CSA_OK;
}

csa_status check_attend(const uint16_t* q, int T, int n_heads, int head_dim, float scale,
                        const uint16_t* kv_a, int64_t a_rows, const uint16_t* kv_b,
                        int64_t b_rows, const int64_t* b_row0, const int32_t* b_len,
                        int max_rows, const uint16_t* out) {
  if (T < 0 || n_heads < 1 || max_rows < 0 || a_rows < 0 || b_rows < 0) return CSA_EINVAL;
  if (!q || !kv_a || !out || !isfinite(scale)) return CSA_EINVAL;
  const bool any_b = kv_b || b_row0 || b_len;
  const bool all_b = kv_b && b_row0 && b_len;
  if (any_b && !all_b) return CSA_EINVAL;
  if (!aligned16(q) || !aligned16(kv_a) || (kv_b && !aligned16(kv_b))) return CSA_EINVAL;
  if (!head_dim_ok(head_dim)) return CSA_EUNSUPPORTED;
  if (n_heads > 128 || T > kMaxGridY) return CSA_EUNSUPPORTED;
  return CSA_OK;
}

csa_status check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return CSA_OK;
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0 || ws_bytes < need)
    return CSA_EWORKSPACE;
  return CSA_OK;
}

// Workspace of a decode step, in carve order.
struct StepWs {
  size_t scores, topk, idx, count, n_kv, attend, pre_idx, pre_count, pre_key, pre_gcut, total;
};

// Keys the step's select holds: four register slots per thread when it runs
// inside the attention kernel (or for a single row), twelve in the select
// kernel of a larger batch -- three times the candidates per group, so that
// the lists of the shorter rows of a ragged batch rarely overflow.
int step_pool(const csa_step_args* a) {
  if (a->T <= 1 || select_attend_fits(a->T, a->n_heads, a->top_k + a->window, kStepSplitTiles))
    return kStepPool;
  return 3 * kStepPool;
}

// Candidates the E4M3 prefilter keeps: half as many again as top_k, at most
// what the select holds in registers.
int prefilter_count(int top_k) {
  const int c = top_k + top_k / 2;
  return c < kStepPool ? c : kStepPool;
}

StepWs step_ws_layout(const csa_step_args* a) {
  StepWs w{};
  size_t off = 0;
  if (a->mode == CSA_MODE_CSA) {
    w.scores = off;
    if (!a->scores) off += align256((size_t)a->T * (size_t)a->max_vis * 4);
    w.topk = off;
    off += topk_ws_layout(nullptr, a->T, plan_topk(a->T, a->max_vis, a->top_k, step_pool(a))).bytes;
    w.idx = off;
    if (!a->idx) off += align256((size_t)a->T * a->top_k * 4);
    w.count = off;
    if (!a->count) off += align256((size_t)a->T * 4);
    w.n_kv = off;
    if (!a->n_kv) off += align256((size_t)a->T * 4);
    w.attend = off;
    const int rows = a->top_k + a->window;
    off += attend_ws_bytes(a->T, a->n_heads, a->head_dim, rows,
                           step_split_tiles(a->T, a->n_heads, rows));
    if (a->idx_e4m3) {
      const size_t C = (size_t)prefilter_count(a->top_k);
      w.pre_idx = off;
      off += align256((size_t)a->T * C * 4);
      w.pre_count = off;
      off += align256((size_t)a->T * 4);
      w.pre_key = off;
      off += align256((size_t)a->T * C * 8);
      w.pre_gcut = off;
      off += align256((size_t)a->T * 8);
    }
  } else {
    w.attend = off;
    const int64_t rows = a->max_vis + a->window;
    off += attend_ws_bytes(a->T, a->n_heads, a->head_dim, rows > INT32_MAX ? INT32_MAX : (int)rows, 0);
  }
  w.total = off;
  return w;
}

csa_status check_step(const csa_step_args* a) {
  if (!a) return CSA_EINVAL;
  if (a->mode != CSA_MODE_CSA && a->mode != CSA_MODE_HCA) return CSA_EINVAL;
  if (a->T < 0 || a->max_vis < 0 || a->window < 0 || a->ratio < 1 || a->n_heads < 1)
    return CSA_EINVAL;
  if (a->comp_rows < 0 || a->swa_rows < 0) return CSA_EINVAL;
  if (!a->q || !a->out || !a->comp_kv || !a->swa || !a->pos || !a->seq_kv || !a->n_comp ||
      !a->swa_row0 || !a->swa_len)
    return CSA_EINVAL;
  if (!isfinite(a->scale)) return CSA_EINVAL;
  if (a->one_sequence != 0 && a->one_sequence != 1) return CSA_EINVAL;
  if (!aligned16(a->q) || !aligned16(a->comp_kv) || !aligned16(a->swa) || !aligned16(a->out))
    return CSA_EINVAL;
  if (!head_dim_ok(a->head_dim) || a->n_heads > 128 || a->T > kMaxGridY || a->window > 1024)
    return CSA_EUNSUPPORTED;
  if (a->max_vis + a->window > INT32_MAX) return CSA_EUNSUPPORTED;
  if (a->mode == CSA_MODE_CSA) {
    if (!a->q_idx || !a->w || !a->k_idx) return CSA_EINVAL;
    if (a->n_ih < 1 || a->top_k < 1 || a->max_vis < 1 || a->k_rows < 0) return CSA_EINVAL;
    if (!aligned16(a->q_idx) || !aligned16(a->k_idx) || (a->all_kv && !aligned16(a->all_kv)) ||
        !aligned4(a->w))
      return CSA_EINVAL;
    if ((a->scores && !aligned16(a->scores)) || (a->idx && !aligned4(a->idx)) ||
        (a->count && !aligned4(a->count)) || (a->n_kv && !aligned4(a->n_kv)))
      return CSA_EINVAL;
    if (a->ihd != 32 && a->ihd != 64 && a->ihd != 128) return CSA_EUNSUPPORTED;
    if (a->n_ih > 128 || a->top_k > kMaxTopk) return CSA_EUNSUPPORTED;
    if (a->idx_e4m3 != 0 && a->idx_e4m3 != 1) return CSA_EINVAL;
    if (a->idx_e4m3 && (!a->q_idx8 || !a->k_idx8 || !a->q_idx_scale || !a->k_idx_scale ||
                        !aligned16(a->q_idx8) || !aligned16(a->k_idx8) ||
                        !aligned4(a->q_idx_scale) || !aligned4(a->k_idx_scale)))
      return CSA_EINVAL;
    if (a->max_vis > INT32_MAX) return CSA_EUNSUPPORTED;
  }
  return CSA_OK;
}

}  // namespace

extern "C" {

const char* csa_status_str(int status) {
  switch (status) {
    case CSA_OK: return "CSA_OK";
    case CSA_EINVAL: return "CSA_EINVAL: invalid argument";
    case CSA_EUNSUPPORTED: return "CSA_EUNSUPPORTED: shape outside the supported set";
    case CSA_EWORKSPACE: return "CSA_EWORKSPACE: workspace missing, misaligned or too small";
    case CSA_EHIP: return "CSA_EHIP: HIP launch failed";
    case CSA_ESCRATCH:
      return "CSA_ESCRATCH: the step needs more workspace than the allocation-free entry "
             "point's fixed scratch (CSA_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown csa_status";
  }
}

int csa_abi_version(void) { return kAbiVersion; }

csa_status csa_index_score(const uint16_t* q_idx, const float* w, const uint16_t* k_idx,
                           int64_t k_rows, const int64_t* pos, const int64_t* seq_kv,
                           const int32_t* n_comp, int T, int n_ih, int ihd, int ratio,
                           float* scores, int64_t ld, uint32_t* err, void* stream) {
  csa_status s = check_index(q_idx, w, k_idx, k_rows, pos, seq_kv, n_comp, T, n_ih, ihd, ratio,
                             scores, ld);
  if (s != CSA_OK || T == 0) return s;
  IndexScoreLaunch L{};
  L.q_idx = q_idx; L.w = w; L.k_idx = k_idx; L.k_rows = k_rows;
  L.pos = pos; L.seq_kv = seq_kv; L.n_comp = n_comp;
  L.T = T; L.n_ih = n_ih; L.ihd = ihd; L.ratio = ratio;
  L.scores = scores; L.ld = ld; L.cand = CandArgs{}; L.err = err;
  return hip_status(launch_index_score(L, static_cast<hipStream_t>(stream)));
}

csa_status csa_index_score_e4m3(const uint8_t* q_idx, const float* q_scale, const float* w,
                                const uint8_t* k_idx, const float* k_scale, int64_t k_rows,
                                const int64_t* pos, const int64_t* seq_kv, const int32_t* n_comp,
                                int T, int n_ih, int ihd, int ratio, float* scores, int64_t ld,
                                uint32_t* err, void* stream) {
  csa_status s = check_index(reinterpret_cast<const uint16_t*>(q_idx), w,
                             reinterpret_cast<const uint16_t*>(k_idx), k_rows, pos, seq_kv, n_comp,
                             T, n_ih, ihd, ratio, scores, ld);
  if (s != CSA_OK) return s;
  if (!q_scale || !k_scale || !aligned4(q_scale) || !aligned4(k_scale)) return CSA_EINVAL;
  if (T == 0) return CSA_OK;
  IndexScoreLaunch L{};
  L.q_idx = q_idx; L.w = w; L.k_idx = k_idx; L.k_rows = k_rows;
  L.e4m3 = 1; L.q_scale = q_scale; L.k_scale = k_scale;
  L.pos = pos; L.seq_kv = seq_kv; L.n_comp = n_comp;
  L.T = T; L.n_ih = n_ih; L.ihd = ihd; L.ratio = ratio;
  L.scores = scores; L.ld = ld; L.cand = CandArgs{}; L.err = err;
  return hip_status(launch_index_score(L, static_cast<hipStream_t>(stream)));
}

csa_status csa_quantize_e4m3(const uint16_t* src, int64_t rows, int d, uint8_t* codes,
                             float* scale, void* stream) {
  if (rows < 0 || d < 1 || !src || !codes || !scale || !aligned4(scale)) return CSA_EINVAL;
  if (d > 512) return CSA_EUNSUPPORTED;
  if (rows == 0) return CSA_OK;
  return hip_status(launch_quant_e4m3(src, rows, d, codes, scale, static_cast<hipStream_t>(stream)));
}

size_t csa_topk_workspace_bytes(int T, int64_t ld, int top_k) {
  if (T <= 0 || ld <= 0 || ld > INT32_MAX || top_k < 1) return 0;
  return topk_ws_layout(nullptr, T, plan_topk(T, ld, top_k, kPoolCap)).bytes;
}

csa_status csa_topk(const float* scores, int64_t ld, const int64_t* pos, const int32_t* n_comp,
                    int T, int ratio, int top_k, int32_t* idx, int32_t* count, void* ws,
                    size_t ws_bytes, uint32_t* err, void* stream) {
  csa_status s = check_topk(scores, ld, pos, n_comp, T, ratio, top_k, idx, count);
  if (s != CSA_OK || T == 0) return s;
  const TopkPlan plan = plan_topk(T, ld, top_k, kPoolCap);
  s = check_ws(ws, ws_bytes, topk_ws_layout(nullptr, T, plan).bytes);
  if (s != CSA_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const TopkWs tw = topk_ws_layout(ws, T, plan);
  hipError_t e = launch_score_cands(scores, ld, pos, n_comp, T, ratio, plan, tw, err, st);
  if (e == hipSuccess)
    e = launch_topk_select(scores, ld, pos, n_comp, nullptr, 0, T, ratio, top_k, plan, tw, idx,
                           count, err, st);
  return hip_status(e);
}

csa_status csa_gather(const uint16_t* comp_kv, int64_t comp_rows, const int64_t* seq_kv,
                      const int32_t* idx, const int32_t* count, int top_k, const uint16_t* swa,
                      int64_t swa_rows, const int64_t* swa_row0, const int32_t* swa_len,
                      int window, int T, int head_dim, uint16_t* all_kv, int32_t* n_kv,
                      uint32_t* err, void* stream) {
  csa_status s = check_gather(comp_kv, comp_rows, seq_kv, idx, count, top_k, swa, swa_rows,
                              swa_row0, swa_len, window, T, head_dim, all_kv, n_kv);
  if (s != CSA_OK || T == 0) return s;
  GatherLaunch L{};
  L.comp_kv = comp_kv; L.comp_rows = comp_rows; L.seq_kv = seq_kv;
  L.idx = idx; L.count = count; L.top_k = top_k;
  L.swa = swa; L.swa_rows = swa_rows; L.swa_row0 = swa_row0; L.swa_len = swa_len;
  L.window = window; L.T = T; L.head_dim = head_dim;
  L.all_kv = all_kv; L.n_kv = n_kv; L.err = err;
  return hip_status(launch_gather(L, static_cast<hipStream_t>(stream)));
}

size_t csa_attend_workspace_bytes(int T, int n_heads, int head_dim, int max_rows) {
  if (T <= 0 || n_heads <= 0 || !head_dim_ok(head_dim) || max_rows < 0) return 0;
  return attend_ws_bytes(T, n_heads, head_dim, max_rows, 0);
}

csa_status csa_mqa_attend(const uint16_t* q, int T, int n_heads, int head_dim, float scale,
                          const float* sink, const uint16_t* kv_a, int64_t a_rows,
                          const int64_t* a_row0, const int32_t* a_len, const uint16_t* kv_b,
                          int64_t b_rows, const int64_t* b_row0, const int32_t* b_len,
                          int max_rows, uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                          uint32_t* err, void* stream) {
  csa_status s = check_attend(q, T, n_heads, head_dim, scale, kv_a, a_rows, kv_b, b_rows, b_row0,
                              b_len, max_rows, out);
  if (s != CSA_OK) return s;
  if (!a_row0 || !a_len) return CSA_EINVAL;
  if (T == 0) return CSA_OK;
  s = check_ws(ws, ws_bytes, attend_ws_bytes(T, n_heads, head_dim, max_rows, 0));
  if (s != CSA_OK) return s;
  AttendLaunch L{};
  L.q = q; L.T = T; L.n_heads = n_heads; L.head_dim = head_dim; L.scale = scale; L.sink = sink;
  L.kv_a = kv_a; L.a_rows = a_rows; L.a_row0 = a_row0; L.a_len = a_len; L.a_stride = 0;
  L.vis_pos = nullptr; L.vis_ncomp = nullptr; L.vis_ratio = 1;
  L.kv_b = kv_b; L.b_rows = b_rows; L.b_row0 = b_row0; L.b_len = b_len;
  L.max_rows = max_rows; L.split_tiles = 0; L.out = out; L.lse = lse; L.ws = ws; L.err = err;
  return hip_status(launch_attend(L, static_cast<hipStream_t>(stream)));
}

size_t csa_decode_step_workspace_bytes(const csa_step_args* a) {
  if (check_step(a) != CSA_OK) return 0;
  return step_ws_layout(a).total;
}

}  // extern "C"

namespace {

// The decode step's stages: kStageIndex (S1 and its candidate lists) and
// kStageRest (S2 .. S4, reading what S1 left in the workspace).
constexpr int kStageIndex = 1, kStageRest = 2;

csa_status run_step(const csa_step_args* a, void* ws, size_t ws_bytes, void* stream, int stages) {
  csa_status s = check_step(a);
  if (s != CSA_OK) return s;
  if (a->T == 0) return CSA_OK;
  const StepWs lay = step_ws_layout(a);
  s = check_ws(ws, ws_bytes, lay.total);
  if (s != CSA_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);

  AttendLaunch L{};
  L.q = a->q; L.T = a->T; L.n_heads = a->n_heads; L.head_dim = a->head_dim;
  L.scale = a->scale; L.sink = a->sink; L.out = a->out; L.lse = a->lse;
  L.ws = base + lay.attend; L.err = a->err;

  if (a->mode == CSA_MODE_HCA) {
    if (!(stages & kStageRest)) return CSA_OK;
    L.kv_a = a->comp_kv; L.a_rows = a->comp_rows; L.a_row0 = a->seq_kv; L.a_len = nullptr;
    L.a_stride = 0; L.vis_pos = a->pos; L.vis_ncomp = a->n_comp; L.vis_ratio = a->ratio;
    L.kv_b = a->swa; L.b_rows = a->swa_rows; L.b_row0 = a->swa_row0; L.b_len = a->swa_len;
    L.max_rows = (int)(a->max_vis + a->window);
    L.split_tiles = 0;
    return hip_status(launch_attend(L, st));
  }

  float* scores = a->scores ? a->scores : reinterpret_cast<float*>(base + lay.scores);
  int32_t* idx = a->idx ? a->idx : reinterpret_cast<int32_t*>(base + lay.idx);
  int32_t* count = a->count ? a->count : reinterpret_cast<int32_t*>(base + lay.count);
  int32_t* n_kv = a->n_kv ? a->n_kv : reinterpret_cast<int32_t*>(base + lay.n_kv);
  const TopkPlan tp = plan_topk(a->T, a->max_vis, a->top_k, step_pool(a));
  const TopkWs tw = topk_ws_layout(base + lay.topk, a->T, tp);

  // S1 with its candidate lists
  IndexScoreLaunch I{};
  I.w = a->w; I.k_rows = a->k_rows;
  if (a->idx_e4m3) {
    I.q_idx = a->q_idx8; I.k_idx = a->k_idx8;
    I.e4m3 = 1; I.q_scale = a->q_idx_scale; I.k_scale = a->k_idx_scale;
  } else {
    I.q_idx = a->q_idx; I.k_idx = a->k_idx;
  }
  I.pos = a->pos; I.seq_kv = a->seq_kv; I.n_comp = a->n_comp;
  I.T = a->T; I.n_ih = a->n_ih; I.ihd = a->ihd; I.ratio = a->ratio;
  I.one_seq = a->one_sequence;
  I.scores = scores; I.ld = a->max_vis;
  I.cand = cand_args(tp, tw); I.err = a->err;
  hipError_t e = hipSuccess;
  if (stages & kStageIndex) {
    e = launch_index_score(I, st);
    if (e != hipSuccess) return hip_status(e);
  }
  if (!(stages & kStageRest)) return CSA_OK;
  // S2, then S3 fused into S4: the selected compressed rows are read through
  // their block indices and the SWA rows in place (and copied into all_kv
  // when it is given)
  L.kv_a = a->comp_kv; L.a_rows = a->comp_rows; L.a_row0 = a->seq_kv; L.a_len = nullptr;
  L.a_stride = 0; L.vis_pos = nullptr; L.vis_ncomp = nullptr; L.vis_ratio = 1;
  L.sel_idx = idx; L.sel_cnt = count; L.sel_stride = a->top_k;
  L.kv_b = a->swa; L.b_rows = a->swa_rows; L.b_row0 = a->swa_row0; L.b_len = a->swa_len;
  L.b_cap = a->window;
  L.copy_out = a->all_kv; L.copy_stride = a->top_k + a->window; L.n_kv_out = n_kv;
  L.max_rows = a->top_k + a->window;
  L.split_tiles = step_split_tiles(a->T, a->n_heads, L.max_rows);
  SelectLaunch S{};
  S.scores = scores; S.ld = a->max_vis; S.pos = a->pos; S.n_comp = a->n_comp;
  S.seq_kv = a->seq_kv; S.k_rows = a->k_rows;
  S.ratio = a->ratio; S.top_k = a->top_k;
  S.cand = tw.cand; S.gcut = tw.gcut; S.list_len = tp.list_len;
  S.groups_per_token = tp.groups_per_token; S.blocks_per_group = tp.blocks_per_group;
  S.idx = idx; S.count = count; S.err = a->err;
  S.row0_group = gemm_indexer(I) ? kGemmTokens : 0;
  if (a->idx_e4m3) {
    // E4M3 prefilter: the C best blocks by E4M3 score, rescored in bf16; they
    // form one complete candidate list per token for the top-k below
    const int C = prefilter_count(a->top_k);
    SelectLaunch P = S;
    P.top_k = C;
    P.idx = reinterpret_cast<int32_t*>(base + lay.pre_idx);
    P.count = reinterpret_cast<int32_t*>(base + lay.pre_count);
    RescoreLaunch R{};
    R.q_idx = a->q_idx; R.w = a->w; R.k_idx = a->k_idx; R.seq_kv = a->seq_kv;
    R.idx = P.idx; R.count = P.count;
    R.T = a->T; R.n_ih = a->n_ih; R.ihd = a->ihd; R.C = C;
    R.key = reinterpret_cast<uint64_t*>(base + lay.pre_key);
    R.gcut = reinterpret_cast<uint64_t*>(base + lay.pre_gcut);
    if (prefilter_rescore_fits(R)) {
      e = launch_prefilter_rescore(P, R, a->T, st);
      if (e != hipSuccess) return hip_status(e);
    } else {
      e = launch_step_select(P, a->T, st);
      if (e != hipSuccess) return hip_status(e);
      e = launch_rescore(R, st);
      if (e != hipSuccess) return hip_status(e);
    }
    S.cand = R.key; S.gcut = R.gcut; S.list_len = C;
    S.groups_per_token = 1; S.blocks_per_group = (int)a->max_vis; S.lists_complete = 1;
  }
  if (select_attend_fits(a->T, a->n_heads, L.max_rows, L.split_tiles))
    return hip_status(launch_select_attend(S, L, st));
  e = launch_step_select(S, a->T, st);
  if (e == hipSuccess) e = launch_attend(L, st);
  return hip_status(e);
}

}  // namespace

extern "C" {

csa_status csa_decode_step(const csa_step_args* a, void* ws, size_t ws_bytes, void* stream) {
  return run_step(a, ws, ws_bytes, stream, kStageIndex | kStageRest);
}

csa_status csa_decode_step_stage(const csa_step_args* a, int stage, void* ws, size_t ws_bytes,
                                 void* stream) {
  if (stage != CSA_STAGE_INDEX && stage != CSA_STAGE_REST) return CSA_EINVAL;
  return run_step(a, ws, ws_bytes, stream, stage == CSA_STAGE_INDEX ? kStageIndex : kStageRest);
}

csa_status csa_decode_step_noalloc(const csa_step_args* a, void* stream) {
  csa_status s = check_step(a);
  if (s != CSA_OK) return s;
  if (a->T == 0) return CSA_OK;
  if (step_ws_layout(a).total > (size_t)CSA_NOALLOC_SCRATCH_BYTES) return CSA_ESCRATCH;
  void* ws = nullptr;
  s = scratch_address(&ws);
  if (s != CSA_OK) return s;
  return csa_decode_step(a, ws, (size_t)CSA_NOALLOC_SCRATCH_BYTES, stream);
}

size_t csa_compress_append_workspace_bytes(int T, int H, int hd, int ihd) {
  if (T <= 0 || H <= 0 || hd <= 0 || ihd <= 0) return 0;
  return compress_ws_bytes(T, H, hd, ihd);
}

csa_status csa_compress_append(const uint16_t* x, int T, int H, const uint16_t* w_kv, int hd,
                               const uint16_t* w_ik, int ihd, const int32_t* seq,
                               const int64_t* pos, int S, int ratio, int window, float* ring,
                               uint16_t* swa, int32_t* swa_head, int32_t* swa_len,
                               uint16_t* comp_kv, uint16_t* k_idx, const int64_t* seq_kv,
                               int32_t* n_comp, int64_t comp_rows, void* ws, size_t ws_bytes,
                               uint32_t* err, void* stream) {
  if (T < 0 || H < 1 || hd < 1 || ihd < 1 || S < 1 || ratio < 1 || window < 1 || comp_rows < 0)
    return CSA_EINVAL;
  if (!x || !w_kv || !w_ik || !seq || !pos || !ring || !swa || !swa_head || !swa_len ||
      !comp_kv || !k_idx || !seq_kv || !n_comp)
    return CSA_EINVAL;
  if (!aligned16(x) || !aligned16(w_kv) || !aligned16(w_ik) || !aligned4(ring) ||
      !aligned4(seq) || !aligned4(swa_head) || !aligned4(swa_len) || !aligned4(n_comp))
    return CSA_EINVAL;
  if (H % 256 != 0 || hd % 16 != 0 || ihd % 16 != 0 || hd > 1024 || ihd > 512 ||
      (ratio & (ratio - 1)) != 0 || ratio > 16 || window > 1024 || T > kMaxGridY * 32)
    return CSA_EUNSUPPORTED;
  if (T == 0) return CSA_OK;
  csa_status st = check_ws(ws, ws_bytes, compress_ws_bytes(T, H, hd, ihd));
  if (st != CSA_OK) return st;
  CompressLaunch c{};
  c.x = x; c.T = T; c.H = H; c.w_kv = w_kv; c.hd = hd; c.w_ik = w_ik; c.ihd = ihd;
  c.seq = seq; c.pos = pos; c.S = S; c.ratio = ratio; c.window = window;
  c.ring = ring; c.swa = swa; c.swa_head = swa_head; c.swa_len = swa_len;
  c.comp_kv = comp_kv; c.k_idx = k_idx; c.seq_kv = seq_kv; c.n_comp = n_comp;
  c.comp_rows = comp_rows; c.ws = ws; c.err = err;
  return hip_status(launch_compress_append(c, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
