// The C ABI of libmoe (declared and documented in include/moe.h): argument checks,
// workspace planning, and the stream-ordered launch sequence of the block.
#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/moe.h"
#include "kernels.h"

// The workspace of moe_forward_static: one copy per device, held until the process ends.
static __device__ __align__(256) uint8_t scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  moe_ws_layout pub;
  size_t meta, blk, tiles_s, tiles_w, tiles_w2, zpart;
  int nsplit;
};

bool aligned16(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

moe_status check_config(const moe_config* c, int64_t T, moe::Dims* d) {
  if (!c) return fail(MOE_ERR_ARG, "cfg is NULL");
  if (T < 0) return fail(MOE_ERR_ARG, "T < 0");
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16 && c->dtype != MOE_FP8)
    return fail(MOE_ERR_CONFIG, "unknown dtype");
  if (c->score_func != MOE_SCORE_SIGMOID && c->score_func != MOE_SCORE_SOFTMAX)
    return fail(MOE_ERR_CONFIG, "unknown score_func");
  if (c->dim <= 0 || c->n_experts <= 0 || c->n_groups <= 0 || c->topk_groups <= 0 || c->topk <= 0 ||
      c->inter <= 0 || c->n_shared <= 0)
    return fail(MOE_ERR_CONFIG, "every size in cfg must be positive");
  if (c->n_experts % c->n_groups) return fail(MOE_ERR_CONFIG, "n_experts must be a multiple of n_groups");
  if (c->topk_groups > c->n_groups) return fail(MOE_ERR_CONFIG, "topk_groups > n_groups");
  if ((int64_t)c->topk > (int64_t)c->topk_groups * (c->n_experts / c->n_groups))
    return fail(MOE_ERR_CONFIG, "topk exceeds the experts of the kept groups");
  if (!(c->route_scale == c->route_scale)) return fail(MOE_ERR_CONFIG, "route_scale is NaN");
  if (c->n_experts > 1024 || c->n_groups > 64 || c->topk > 16)
    return fail(MOE_ERR_UNSUPPORTED, "kernels handle n_experts <= 1024, n_groups <= 64, topk <= 16");
  const int64_t S = (int64_t)c->n_shared * c->inter;
  if (c->dtype == MOE_BF16 && (c->dim % 128 || c->inter % 32 || S % 32))
    return fail(MOE_ERR_UNSUPPORTED, "bf16 needs dim % 128 == 0 and inter % 32 == 0");
  if (c->dtype == MOE_FP8 && (c->dim % 128 || c->inter % 128))
    return fail(MOE_ERR_UNSUPPORTED, "fp8 needs dim and inter multiples of 128");
  if ((int64_t)T * c->topk >= (int64_t)1 << 31 || T * (int64_t)c->dim >= (int64_t)1 << 40)
    return fail(MOE_ERR_UNSUPPORTED, "too many tokens");
  d->T = T;
  d->R = T * c->topk;
  d->D = c->dim;
  d->E = c->n_experts;
  d->G = c->n_groups;
  d->Gk = c->topk_groups;
  d->K = c->topk;
  d->I = c->inter;
  d->S = (int)S;
  d->dtype = c->dtype;
  return MOE_OK;
}

Layout plan(const moe::Dims& d) {
  Layout L;
  memset(&L, 0, sizeof(L));
  const size_t act = d.dtype == MOE_F32 ? 4 : d.dtype == MOE_BF16 ? 2 : 1;
  const size_t outb = d.dtype == MOE_F32 ? 4 : 2;
  const bool fp8 = d.dtype == MOE_FP8;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  L.pub.idx = take(d.R * 4);
  L.pub.w = take(d.R * 4);
  L.pub.counts = take((size_t)d.E * 4);
  L.pub.offsets = take(((size_t)d.E + 1) * 4);
  L.pub.row_token = take(d.R * 4);
  L.pub.row_of = take(d.R * 4);
  L.meta = take(moe::kMetaInts * 4);
  L.blk = take((size_t)std::max(1, moe::dispatch_blocks(d.T)) * d.E * 4);
  L.tiles_s = take((size_t)moe::max_tiles(d, moe::kSkinnyBM) * sizeof(Tile));
  L.tiles_w = take((size_t)moe::max_tiles(d, moe::kWideBM) * sizeof(Tile));
  L.tiles_w2 = take((size_t)moe::max_tiles(d, moe::kWideBM2) * sizeof(Tile));
  L.nsplit = moe::router_splits(d);
  L.zpart = take((size_t)L.nsplit * d.T * d.E * 8);
  L.pub.xq = take(fp8 ? (size_t)d.T * d.D : 0);
  L.pub.x_scale = take(fp8 ? (size_t)d.T * (d.D / 128) * 4 : 0);
  L.pub.h_routed = take((size_t)d.R * d.I * act);
  L.pub.h_shared = take((size_t)d.T * d.S * act);
  L.pub.h_scale = take(fp8 ? (size_t)d.R * (d.I / 128) * 4 : 0);
  L.pub.h_shared_scale = take(fp8 ? (size_t)d.T * (d.S / 128) * 4 : 0);
  L.pub.o_routed = take((size_t)d.R * d.D * outb);
  L.pub.o_shared = take((size_t)d.T * d.D * outb);
  L.pub.total = o;
  return L;
}

// A dense feed-forward as a block with no routed experts: E = 0, K = 0, the shared expert of
// width S = inter on every token (I = S as well, so kernels that take S == I accept it).
moe_status check_ffn_config(const moe_ffn_config* c, int64_t T, moe::Dims* d) {
  if (!c) return fail(MOE_ERR_ARG, "cfg is NULL");
  if (T < 0) return fail(MOE_ERR_ARG, "T < 0");
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16 && c->dtype != MOE_FP8)
    return fail(MOE_ERR_CONFIG, "unknown dtype");
  if (c->dim <= 0 || c->inter <= 0) return fail(MOE_ERR_CONFIG, "dim and inter must be positive");
  if (c->dtype == MOE_BF16 && (c->dim % 128 || c->inter % 32))
    return fail(MOE_ERR_UNSUPPORTED, "bf16 needs dim % 128 == 0 and inter % 32 == 0");
  if (c->dtype == MOE_FP8 && (c->dim % 128 || c->inter % 128))
    return fail(MOE_ERR_UNSUPPORTED, "fp8 needs dim and inter multiples of 128");
  if (T >= (int64_t)1 << 31 || T * (int64_t)c->dim >= (int64_t)1 << 40 || T * (int64_t)c->inter >= (int64_t)1 << 40)
    return fail(MOE_ERR_UNSUPPORTED, "too many tokens");
  d->T = T;
  d->R = 0;
  d->D = c->dim;
  d->E = 0;
  d->G = 1;
  d->Gk = 1;
  d->K = 0;
  d->I = c->inter;
  d->S = c->inter;
  d->dtype = c->dtype;
  return MOE_OK;
}

// Workspace of the dense feed-forward: tile lists, x's fp8 image, h (+ scales). The down GEMM
// writes the output itself.
Layout plan_ffn(const moe::Dims& d) {
  Layout L;
  memset(&L, 0, sizeof(L));
  const size_t act = d.dtype == MOE_F32 ? 4 : d.dtype == MOE_BF16 ? 2 : 1;
  const bool fp8 = d.dtype == MOE_FP8;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  L.pub.offsets = take(4);
  L.meta = take(moe::kMetaInts * 4);
  L.tiles_s = take((size_t)moe::max_tiles(d, moe::kSkinnyBM) * sizeof(Tile));
  L.tiles_w = take((size_t)moe::max_tiles(d, moe::kWideBM) * sizeof(Tile));
  L.tiles_w2 = take((size_t)moe::max_tiles(d, moe::kWideBM2) * sizeof(Tile));
  L.pub.xq = take(fp8 ? (size_t)d.T * d.D : 0);
  L.pub.x_scale = take(fp8 ? (size_t)d.T * (d.D / 128) * 4 : 0);
  L.pub.h_shared = take((size_t)d.T * d.S * act);
  L.pub.h_shared_scale = take(fp8 ? (size_t)d.T * (d.S / 128) * 4 : 0);
  const int split = moe::dense_down_split(d);
  L.zpart = take(split > 1 ? (size_t)split * d.T * d.D * 4 : 0);  // the down projection's partial sums
  L.pub.total = o;
  return L;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

moe_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

moe_status check_ws(const Layout& L, const void* ws, size_t ws_bytes) {
  if (ws_bytes < L.pub.total)
    return fail(MOE_ERR_WORKSPACE, "workspace of " + std::to_string(ws_bytes) + " bytes, need " +
                                       std::to_string(L.pub.total));
  if (!ws && L.pub.total) return fail(MOE_ERR_ARG, "ws is NULL");
  if (!aligned16(ws)) return fail(MOE_ERR_ARG, "ws is not 16-byte aligned");
  return MOE_OK;
}

// ---- the allocation-free forward (moe_forward_static): one workspace per device in the
// file-scope device array `scratch` (declared above the anonymous namespace). In host code
// `scratch` names a host-side stand-in; the device address comes from hipGetSymbolAddress, once
// per device with that device current, and only that address is used.
std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_at;  // device -> address of that device's copy of `scratch`

moe_status static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch_at.find(dev);
  if (it == g_scratch_at.end()) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MOE_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    it = g_scratch_at.emplace(dev, p).first;
  }
  *ptr = it->second;
  return MOE_OK;
}

// ---- measurement spans (moe_timing_enable / moe_timing_report)
struct SpanRec {
  const char* name;
  hipEvent_t a, b;
};
std::mutex g_tmu;
bool g_timing = false;
std::string g_filter;  // record only kernels whose name contains this ("" = all)
std::vector<hipEvent_t> g_pool;
std::vector<SpanRec> g_spans;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void drop_spans() {
  for (auto& r : g_spans) {
    if (r.a) g_pool.push_back(r.a);
    if (r.b) g_pool.push_back(r.b);
  }
  g_spans.clear();
}

}  // namespace

namespace moe {
int device_lds_limit() {
  static std::mutex mu;
  static std::map<int, int> cache;  // device -> per-block LDS limit
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lk(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) v = 0;
  cache[dev] = v;
  return v;
}

hipError_t allow_dynamic_lds(const void* kernel, size_t bytes) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, hipError_t> done;  // (device, kernel) -> result
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(mu);
  auto key = std::make_pair(dev, kernel);
  auto it = done.find(key);
  if (it != done.end()) return it->second;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  done[key] = e;
  return e;
}

int persistent_grid(const void* kernel, int threads, size_t dyn_lds, int max_per_cu) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, std::pair<int, int>> cache;  // (blocks per CU, CUs)
  int dev = 0;
  (void)hipGetDevice(&dev);
  std::lock_guard<std::mutex> lk(mu);
  auto key = std::make_pair(dev, kernel);
  auto it = cache.find(key);
  if (it == cache.end()) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, dyn_lds) != hipSuccess || per_cu < 1)
      per_cu = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    it = cache.emplace(key, std::make_pair(per_cu, cus)).first;
  }
  const int per_cu = max_per_cu > 0 ? std::min(max_per_cu, it->second.first) : it->second.first;
  return per_cu * it->second.second;
}

bool span_begin(const char* name, hipStream_t s) {
  if (!g_timing) return false;
  std::lock_guard<std::mutex> lk(g_tmu);
  if (!g_filter.empty() && !strstr(name, g_filter.c_str())) return false;
  SpanRec r{name, take_event(), nullptr};
  if (r.a) (void)hipEventRecord(r.a, s);
  g_spans.push_back(r);
  return true;
}
void span_end(hipStream_t s) {
  if (!g_timing) return;
  std::lock_guard<std::mutex> lk(g_tmu);
  if (g_spans.empty() || g_spans.back().b) return;
  hipEvent_t e = take_event();
  if (e) (void)hipEventRecord(e, s);
  g_spans.back().b = e;
}
}  // namespace moe

extern "C" {

moe_status moe_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_tmu);
  drop_spans();
  if (on) {
    // make sure events can be created before claiming success
    hipEvent_t e = take_event();
    if (!e) return fail(MOE_ERR_HIP, "hipEventCreate failed");
    g_pool.push_back(e);
  }
  g_timing = on != 0;
  return MOE_OK;
}

moe_status moe_timing_filter(const char* name_part) {
  std::lock_guard<std::mutex> lk(g_tmu);
  g_filter = name_part ? name_part : "";
  return MOE_OK;
}

int moe_timing_report(char* buf, size_t bytes) {
  std::lock_guard<std::mutex> lk(g_tmu);
  std::map<std::string, std::pair<long, double>> acc;
  std::vector<std::string> order;
  for (auto& r : g_spans) {
    if (!r.a || !r.b) continue;
    if (hipEventSynchronize(r.b) != hipSuccess) {
      drop_spans();
      return fail(MOE_ERR_HIP, "hipEventSynchronize failed");
    }
    float ms = 0.f;
    (void)hipEventElapsedTime(&ms, r.a, r.b);
    auto it = acc.find(r.name);
    if (it == acc.end()) {
      order.push_back(r.name);
      acc[r.name] = {1, ms};
    } else {
      it->second.first += 1;
      it->second.second += ms;
    }
  }
  drop_spans();
  std::string out;
  for (auto& n : order) {
    char line[256];
    snprintf(line, sizeof(line), "%s %ld %.6f\n", n.c_str(), acc[n].first, acc[n].second);
    out += line;
  }
  if (buf && bytes) {
    size_t n = std::min(bytes - 1, out.size());
    memcpy(buf, out.data(), n);
    buf[n] = 0;
  }
  return (int)order.size();
}

moe_status moe_workspace_size(const moe_config* cfg, int64_t T, size_t* bytes) {
  moe::Dims d;
  if (!bytes) return fail(MOE_ERR_ARG, "bytes is NULL");
  moe_status st = check_config(cfg, T, &d);
  if (st != MOE_OK) return st;
  *bytes = plan(d).pub.total;
  return MOE_OK;
}

moe_status moe_workspace_layout(const moe_config* cfg, int64_t T, moe_ws_layout* layout) {
  moe::Dims d;
  if (!layout) return fail(MOE_ERR_ARG, "layout is NULL");
  moe_status st = check_config(cfg, T, &d);
  if (st != MOE_OK) return st;
  *layout = plan(d).pub;
  return MOE_OK;
}

moe_status moe_route(const moe_config* cfg, const void* w_gate, const float* bias, const void* x, int64_t T,
                     int32_t* idx, float* w, void* ws, size_t ws_bytes, void* stream) {
  moe::Dims d;
  moe_status st = check_config(cfg, T, &d);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!w_gate || !x || !idx || !w) return fail(MOE_ERR_ARG, "NULL tensor argument");
  if (!aligned16(w_gate) || !aligned16(x) || !aligned16(bias) || !aligned16(idx) || !aligned16(w))
    return fail(MOE_ERR_ARG, "device pointers must be 16-byte aligned");
  if (bias && d.G > 1 && d.E / d.G < 2) return fail(MOE_ERR_CONFIG, "top-2 group score needs 2 experts per group");
  Layout L = plan(d);
  if ((st = check_ws(L, ws, ws_bytes)) != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  double* zpart = at<double>(ws, L.zpart);
  if ((st = hip_status(moe::launch_router_logits(d, x, w_gate, zpart, L.nsplit, s), "router logits")) != MOE_OK)
    return st;
  return hip_status(moe::launch_router_select(d, zpart, L.nsplit, bias, cfg->route_scale, cfg->score_func == MOE_SCORE_SOFTMAX, idx, w, s),
                    "router select");
}

moe_status moe_dispatch(const moe_config* cfg, const int32_t* idx, int64_t T, int32_t* counts, int32_t* offsets,
                        int32_t* row_token, int32_t* row_of, void* ws, size_t ws_bytes, void* stream) {
  moe::Dims d;
  moe_status st = check_config(cfg, T, &d);
  if (st != MOE_OK) return st;
  if (!counts || !offsets || (T > 0 && (!idx || !row_token || !row_of)))
    return fail(MOE_ERR_ARG, "NULL tensor argument");
  Layout L = plan(d);
  if ((st = check_ws(L, ws, ws_bytes)) != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(moe::launch_dispatch(d, idx, at<int32_t>(ws, L.blk), counts, offsets, row_token, row_of,
                                         at<int32_t>(ws, L.meta), at<Tile>(ws, L.tiles_s),
                                         at<Tile>(ws, L.tiles_w), at<Tile>(ws, L.tiles_w2), s),
                    "dispatch");
}

}  // extern "C"

namespace {
// The host-side checks of a block forward (T > 0): tensors present and aligned, configuration,
// workspace size.
moe_status check_forward(const moe_config* cfg, const moe_weights* wts, const void* x, const void* out,
                         const moe::Dims& d, const Layout& L, const void* ws, size_t ws_bytes) {
  if (!x || !out || !wts->w_gate || !wts->w1 || !wts->w3 || !wts->w2 || !wts->ws1 || !wts->ws3 || !wts->ws2)
    return fail(MOE_ERR_ARG, "NULL tensor argument");
  if (d.dtype == MOE_FP8 && (!wts->s1 || !wts->s3 || !wts->s2 || !wts->ss1 || !wts->ss3 || !wts->ss2))
    return fail(MOE_ERR_ARG, "fp8 weights need their block scales");
  const void* ptrs[] = {x, out, wts->w_gate, wts->bias, wts->w1, wts->w3, wts->w2, wts->ws1, wts->ws3, wts->ws2};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(MOE_ERR_ARG, "device pointers must be 16-byte aligned");
  if (wts->bias && d.G > 1 && d.E / d.G < 2)
    return fail(MOE_ERR_CONFIG, "top-2 group score needs 2 experts per group");
  return check_ws(L, ws, ws_bytes);
}

// The expert-GEMM view of a forward workspace.
moe::Act forward_act(const moe::Dims& d, const Layout& L, const void* x, void* ws) {
  const bool fp8 = d.dtype == MOE_FP8;
  moe::Act act;
  act.x = fp8 ? static_cast<const void*>(at<uint8_t>(ws, L.pub.xq)) : x;
  act.x_scale = fp8 ? at<float>(ws, L.pub.x_scale) : nullptr;
  act.row_token = at<int32_t>(ws, L.pub.row_token);
  act.offsets = at<int32_t>(ws, L.pub.offsets);
  act.meta = at<int32_t>(ws, L.meta);
  act.tiles_skinny = at<Tile>(ws, L.tiles_s);
  act.tiles_wide = at<Tile>(ws, L.tiles_w);
  act.tiles_wide2 = at<Tile>(ws, L.tiles_w2);
  act.h_routed = at<void>(ws, L.pub.h_routed);
  act.h_shared = at<void>(ws, L.pub.h_shared);
  act.h_scale = fp8 ? at<float>(ws, L.pub.h_scale) : nullptr;
  act.h_shared_scale = fp8 ? at<float>(ws, L.pub.h_shared_scale) : nullptr;
  act.o_routed = at<void>(ws, L.pub.o_routed);
  act.o_shared = at<void>(ws, L.pub.o_shared);
  return act;
}
}  // namespace

extern "C" {

moe_status moe_forward(const moe_config* cfg, const moe_weights* wts, const void* x, int64_t T, void* out, void* ws,
                       size_t ws_bytes, void* stream) {
  moe::Dims d;
  moe_status st = check_config(cfg, T, &d);
  if (st != MOE_OK) return st;
  if (!wts) return fail(MOE_ERR_ARG, "wts is NULL");
  if (T == 0) return MOE_OK;
  Layout L = plan(d);
  if ((st = check_forward(cfg, wts, x, out, d, L, ws, ws_bytes)) != MOE_OK) return st;
  const bool fp8 = d.dtype == MOE_FP8;
  hipStream_t s = static_cast<hipStream_t>(stream);

  int32_t* idx = at<int32_t>(ws, L.pub.idx);
  float* w = at<float>(ws, L.pub.w);
  int32_t* offsets = at<int32_t>(ws, L.pub.offsets);
  int32_t* row_token = at<int32_t>(ws, L.pub.row_token);
  int32_t* row_of = at<int32_t>(ws, L.pub.row_of);
  int32_t* meta = at<int32_t>(ws, L.meta);
  double* zpart = at<double>(ws, L.zpart);

  if (fp8 && (st = hip_status(moe::launch_act_quant(d, static_cast<const bf16_t*>(x), at<uint8_t>(ws, L.pub.xq),
                                                    at<float>(ws, L.pub.x_scale), s),
                              "activation quantisation")) != MOE_OK)
    return st;
  if ((st = hip_status(moe::launch_router_logits(d, x, wts->w_gate, zpart, L.nsplit, s), "router logits")) != MOE_OK)
    return st;
  if ((st = hip_status(moe::launch_router_select(d, zpart, L.nsplit, wts->bias, cfg->route_scale, cfg->score_func == MOE_SCORE_SOFTMAX, idx,
                                                       w, s),
                       "router select")) != MOE_OK)
    return st;
  if ((st = hip_status(moe::launch_dispatch(d, idx, at<int32_t>(ws, L.blk), at<int32_t>(ws, L.pub.counts), offsets,
                                            row_token, row_of, meta, at<Tile>(ws, L.tiles_s),
                                            at<Tile>(ws, L.tiles_w), at<Tile>(ws, L.tiles_w2), s),
                       "dispatch")) != MOE_OK)
    return st;
  moe::ExpertPtrs ep{wts->w1, wts->w3, wts->w2, wts->ws1, wts->ws3, wts->ws2,
                     wts->s1, wts->s3, wts->s2, wts->ss1, wts->ss3, wts->ss2};
  const moe::Act act = forward_act(d, L, x, ws);
  if ((st = hip_status(moe::launch_experts(d, ep, act, s), "experts")) != MOE_OK) return st;
  return hip_status(moe::launch_combine(d, idx, w, row_of, act.o_routed, act.o_shared, out, s), "combine");
}

moe_status moe_forward_fused(const moe_config* cfg, const moe_weights* wts, const void* x, int64_t T, void* out,
                             void* ws, size_t ws_bytes, void* stream) {
  moe::Dims d;
  moe_status st = check_config(cfg, T, &d);
  if (st != MOE_OK) return st;
  if (!wts) return fail(MOE_ERR_ARG, "wts is NULL");
  if (T == 0) return MOE_OK;
  if (!moe::decode_fused_ok(d))
    return fail(MOE_ERR_UNSUPPORTED, "the fused decode takes bf16 blocks of 1 to " + std::to_string(moe::kFusedMaxT) +
                                         " tokens and at most " + std::to_string(moe::kFusedMaxE) + " experts");
  Layout L = plan(d);
  if ((st = check_forward(cfg, wts, x, out, d, L, ws, ws_bytes)) != MOE_OK) return st;
  moe::ExpertPtrs ep{wts->w1, wts->w3, wts->w2, wts->ws1, wts->ws3, wts->ws2,
                     nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  const moe::Act act = forward_act(d, L, x, ws);
  return hip_status(moe::launch_decode_fused(d, ep, wts->w_gate, wts->bias, cfg->route_scale,
                                             cfg->score_func == MOE_SCORE_SOFTMAX, x, at<double>(ws, L.zpart), L.nsplit,
                                             at<int32_t>(ws, L.pub.idx), at<float>(ws, L.pub.w),
                                             at<int32_t>(ws, L.pub.counts), act, at<int32_t>(ws, L.pub.row_of), out,
                                             static_cast<hipStream_t>(stream)),
                    "fused decode");
}

moe_status moe_forward_static(const moe_config* cfg, const moe_weights* wts, const void* x, int64_t T, void* out,
                              void* stream) {
  moe::Dims d;
  moe_status st = check_config(cfg, T, &d);
  if (st != MOE_OK) return st;
  const size_t need = plan(d).pub.total;
  if (need > (size_t)MOE_STATIC_SCRATCH_BYTES)
    return fail(MOE_ERR_UNSUPPORTED, "T = " + std::to_string(T) + " needs " + std::to_string(need) +
                                         " bytes of workspace; the static scratch holds " +
                                         std::to_string((size_t)MOE_STATIC_SCRATCH_BYTES) +
                                         " (use moe_forward with a caller workspace)");
  if (T == 0) return wts ? MOE_OK : fail(MOE_ERR_ARG, "wts is NULL");
  void* ws = nullptr;
  if ((st = static_scratch(&ws)) != MOE_OK) return st;
  return moe_forward(cfg, wts, x, T, out, ws, (size_t)MOE_STATIC_SCRATCH_BYTES, stream);
}

moe_status moe_ffn_workspace_size(const moe_ffn_config* cfg, int64_t T, size_t* bytes) {
  moe::Dims d;
  if (!bytes) return fail(MOE_ERR_ARG, "bytes is NULL");
  moe_status st = check_ffn_config(cfg, T, &d);
  if (st != MOE_OK) return st;
  *bytes = plan_ffn(d).pub.total;
  return MOE_OK;
}

moe_status moe_ffn(const moe_ffn_config* cfg, const moe_ffn_weights* wts, const void* x, int64_t T, void* out,
                   void* ws, size_t ws_bytes, void* stream) {
  moe::Dims d;
  moe_status st = check_ffn_config(cfg, T, &d);
  if (st != MOE_OK) return st;
  if (!wts) return fail(MOE_ERR_ARG, "wts is NULL");
  if (T == 0) return MOE_OK;
  if (!x || !out || !wts->w1 || !wts->w3 || !wts->w2) return fail(MOE_ERR_ARG, "NULL tensor argument");
  const bool fp8 = d.dtype == MOE_FP8;
  if (fp8 && (!wts->s1 || !wts->s3 || !wts->s2)) return fail(MOE_ERR_ARG, "fp8 weights need their block scales");
  const void* ptrs[] = {x, out, wts->w1, wts->w3, wts->w2, wts->s1, wts->s3, wts->s2};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(MOE_ERR_ARG, "device pointers must be 16-byte aligned");
  Layout L = plan_ffn(d);
  if ((st = check_ws(L, ws, ws_bytes)) != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);

  int32_t* offsets = at<int32_t>(ws, L.pub.offsets);
  int32_t* meta = at<int32_t>(ws, L.meta);
  if (fp8 && (st = hip_status(moe::launch_act_quant(d, static_cast<const bf16_t*>(x), at<uint8_t>(ws, L.pub.xq),
                                                    at<float>(ws, L.pub.x_scale), s),
                              "activation quantisation")) != MOE_OK)
    return st;
  if ((st = hip_status(moe::launch_dense_tiles(d, offsets, meta, at<Tile>(ws, L.tiles_s), at<Tile>(ws, L.tiles_w),
                                               at<Tile>(ws, L.tiles_w2), s),
                       "tile lists")) != MOE_OK)
    return st;
  // the weights take the shared expert's place; there are no routed rows
  moe::ExpertPtrs ep{nullptr, nullptr, nullptr, wts->w1, wts->w3, wts->w2,
                     nullptr, nullptr, nullptr, wts->s1, wts->s3, wts->s2};
  moe::Act act;
  act.x = fp8 ? static_cast<const void*>(at<uint8_t>(ws, L.pub.xq)) : x;
  act.x_scale = fp8 ? at<float>(ws, L.pub.x_scale) : nullptr;
  act.row_token = nullptr;
  act.offsets = offsets;
  act.meta = meta;
  act.tiles_skinny = at<Tile>(ws, L.tiles_s);
  act.tiles_wide = at<Tile>(ws, L.tiles_w);
  act.tiles_wide2 = at<Tile>(ws, L.tiles_w2);
  act.h_routed = nullptr;
  act.h_shared = at<void>(ws, L.pub.h_shared);
  act.h_scale = nullptr;
  act.h_shared_scale = fp8 ? at<float>(ws, L.pub.h_shared_scale) : nullptr;
  act.o_routed = nullptr;
  act.o_shared = out;  // the down GEMM's shared-expert output is the result, in x's dtype
  act.part = moe::dense_down_split(d) > 1 ? at<float>(ws, L.zpart) : nullptr;
  return hip_status(moe::launch_experts(d, ep, act, s), "dense feed-forward");
}

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_ARG: return "invalid argument";
    case MOE_ERR_CONFIG: return "invalid configuration";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP error";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    default: return "unknown status";
  }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
