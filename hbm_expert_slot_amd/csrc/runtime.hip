// Host runtime of libslotcache: configuration checks, buffer layout, the
// exact-size pinned backing store, step enqueue and state readback.
//
// Allocation discipline follows the page "GLM 5.3 Testing: HBM Expert
// Allocation" (section "Five launches, four failures"): pinned host memory is
// requested at the exact byte size (a power-of-two rounding allocator wasted a
// third of host memory there), and every device buffer is sized up front by
// the caller from slotcache_query_sizes (no allocation after start-up).
#include "internal.h"

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

using namespace sc;

// Per-call scratch of moe_layer_decode_static, for callers that cannot
// allocate: one fixed array per GPU, held until the process ends.  Host code
// never uses this name as an address (on the host it is only a stand-in for
// the symbol): the device address comes from hipGetSymbolAddress, looked up
// once per device (static_scratch below).
static __device__ __align__(256) uint8_t scratch[SC_STATIC_SCRATCH_BYTES];

namespace {

thread_local std::string g_err;

sc_status fail(sc_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

sc_status hip_fail(hipError_t e, const char* what) {
  return fail(SC_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
constexpr int64_t kMaxStateStep = (int64_t)1 << 40;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct LayerOffsets {
  size_t e2s, s2e, key, misc, events, end;   // within the layer's state block
};

// misc block: step(8) counters(C_N*8) ev_head(8) error(4)
constexpr size_t kMiscStep = 0;
constexpr size_t kMiscCounters = 8;
constexpr size_t kMiscEvHead = 8 + 8 * C_N;
constexpr size_t kMiscError = kMiscEvHead + 8;
constexpr size_t kMiscBytes = kMiscError + 8;

LayerOffsets layer_offsets(int E, int S, int cap) {
  LayerOffsets o;
  size_t p = 0;
  o.e2s = p; p = align_up(p + (size_t)E * 4);
  o.s2e = p; p = align_up(p + (size_t)S * 4);
  o.key = p; p = align_up(p + (size_t)S * 8);
  o.misc = p; p = align_up(p + kMiscBytes);
  o.events = p; p = align_up(p + (size_t)cap * sizeof(sc_event));
  o.end = p;
  return o;
}

struct WsOffsets {
  size_t hdr, pick_expert, pick_w, pick_u, uniq_expert, uniq_ptr, uniq_off, uniq_picks,
      miss_src, miss_dst, h, part, span, uniq_order, stage, end;
};

// Blocks of a launch whose execution stamps are kept: the GEMV grids are
// capped at 1024 (2048 leaves room), the combine has one block per 256
// outputs.  A larger launch runs without stamps.
int span_blocks(int Pmax_rows, int H) {
  const long comb = ((long)Pmax_rows * H + 255) / 256;
  return (int)(comb > 2048 ? comb : 2048);
}

// Experts the prefill staging area holds (none when no step can be a prefill chunk).
int stage_experts(const sc_config* c) { return c->max_rows > kCachedRows ? c->prefill_stage : 0; }

WsOffsets ws_offsets(int Pmax, int H, int I, int max_rows, int stage_n, int64_t blob) {
  WsOffsets o;
  size_t p = 0;
  o.hdr = p; p = align_up(p + H_WORDS * 4);
  o.pick_expert = p; p = align_up(p + (size_t)Pmax * 4);
  o.pick_w = p; p = align_up(p + (size_t)Pmax * 4);
  o.pick_u = p; p = align_up(p + (size_t)Pmax * 4);
  o.uniq_expert = p; p = align_up(p + (size_t)Pmax * 4);
  o.uniq_ptr = p; p = align_up(p + (size_t)Pmax * 8);
  o.uniq_off = p; p = align_up(p + (size_t)(Pmax + 1) * 4);
  o.uniq_picks = p; p = align_up(p + (size_t)Pmax * 4);
  o.miss_src = p; p = align_up(p + (size_t)Pmax * 8);
  o.miss_dst = p; p = align_up(p + (size_t)Pmax * 8);
  o.h = p; p = align_up(p + (size_t)Pmax * I * 4);
  o.part = p; p = align_up(p + (size_t)Pmax * H * 4);
  o.span = p; p = align_up(p + (size_t)SC_N_KERNELS * span_blocks(max_rows, H) * kSpanSlots * 8);
  o.uniq_order = p; p = align_up(p + (size_t)Pmax * 4);
  o.stage = p; p = align_up(p + (size_t)stage_n * (size_t)blob);
  o.end = p;
  return o;
}

bool supported_hidden(int H) { return gemv_supported(H, true); }
bool supported_inter(int I) { return gemv_supported(I, false); }

sc_status check_config(const sc_config* c) {
  if (!c) return fail(SC_E_ARG, "config is NULL");
  if (c->n_layers < 1) return fail(SC_E_ARG, "n_layers must be >= 1");
  if (c->top_k < 1 || c->top_k > kMaxTopK) return fail(SC_E_ARG, "top_k must be in [1, %d]", kMaxTopK);
  if (c->n_experts < c->top_k || c->n_experts > kMaxExperts)
    return fail(SC_E_ARG, "n_experts must be in [top_k, %d]", kMaxExperts);
  if (c->hidden <= 0 || c->hidden % 64 || c->inter <= 0 || c->inter % 64)
    return fail(SC_E_ARG, "hidden and inter must be positive multiples of 64");
  if (!supported_hidden(c->hidden))
    return fail(SC_E_UNSUPPORTED, "hidden=%d has no compiled gate/up kernel", c->hidden);
  if (!supported_inter(c->inter))
    return fail(SC_E_UNSUPPORTED, "inter=%d has no compiled down kernel", c->inter);
  if (c->max_rows < 1 || c->max_rows > kMaxRows) return fail(SC_E_ARG, "max_rows must be in [1, %d]", kMaxRows);
  if ((long)c->max_rows * c->top_k > kMaxPicks)
    return fail(SC_E_ARG, "max_rows * top_k must be <= %d", kMaxPicks);
  if (c->n_banks < 1 || c->n_banks > c->n_layers) return fail(SC_E_ARG, "n_banks must be in [1, n_layers]");
  if (c->event_capacity < 0) return fail(SC_E_ARG, "event_capacity must be >= 0");
  if (c->flags & ~(uint32_t)(SC_FLAG_BATCH_INVARIANT | SC_FLAG_OVERLAP_FILL))
    return fail(SC_E_ARG, "unknown flags 0x%x", c->flags);
  if (c->prefill_stage < 0 || c->prefill_stage > kMaxExperts)
    return fail(SC_E_ARG, "prefill_stage must be in [0, %d]", kMaxExperts);
  if (!c->slots_per_layer) return fail(SC_E_ARG, "slots_per_layer is NULL");
  for (int l = 0; l < c->n_layers; ++l) {
    int S = c->slots_per_layer[l];
    if (S < 1 || S > c->n_experts || S > kMaxSlots)
      return fail(SC_E_ARG, "slots_per_layer[%d]=%d must be in [1, min(E, %d)]", l, S, kMaxSlots);
  }
  return SC_OK;
}

int ev_cap_of(const sc_config* c) { return c->event_capacity ? c->event_capacity : 4096; }

// Workspace view of a scratch region laid out by `o`.
Workspace bind_workspace(uint8_t* ws, const WsOffsets& o, int stage_n) {
  Workspace W;
  W.hdr = reinterpret_cast<int32_t*>(ws + o.hdr);
  W.pick_expert = reinterpret_cast<int32_t*>(ws + o.pick_expert);
  W.pick_w = reinterpret_cast<float*>(ws + o.pick_w);
  W.pick_u = reinterpret_cast<int32_t*>(ws + o.pick_u);
  W.uniq_expert = reinterpret_cast<int32_t*>(ws + o.uniq_expert);
  W.uniq_ptr = reinterpret_cast<const uint8_t**>(ws + o.uniq_ptr);
  W.uniq_off = reinterpret_cast<int32_t*>(ws + o.uniq_off);
  W.uniq_picks = reinterpret_cast<int32_t*>(ws + o.uniq_picks);
  W.miss_src = reinterpret_cast<const uint8_t**>(ws + o.miss_src);
  W.miss_dst = reinterpret_cast<uint8_t**>(ws + o.miss_dst);
  W.h = reinterpret_cast<float*>(ws + o.h);
  W.part = reinterpret_cast<float*>(ws + o.part);
  W.uniq_order = reinterpret_cast<int32_t*>(ws + o.uniq_order);
  W.stage_n = stage_n;
  W.stage = stage_n > 0 ? ws + o.stage : nullptr;
  return W;
}

// Layout of the static scratch for a configuration: steps of at most
// SC_BYPASS_ROWS rows, no prefill staging area.
WsOffsets static_offsets(const sc_config* c) {
  const int rows = c->max_rows < kCachedRows ? c->max_rows : kCachedRows;
  return ws_offsets(rows * c->top_k, c->hidden, c->inter, rows, 0, 0);
}

// Device address of `scratch` on each device, looked up once per device (with
// that device current) and kept for the life of the process.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch[kMaxDevices];

sc_status static_scratch(int dev, uint8_t** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (dev < 0 || dev >= kMaxDevices) return fail(SC_E_UNSUPPORTED, "device %d beyond the scratch table", dev);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail(SC_E_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    }
    // set-up, not a step: the array starts out zeroed once, before any call uses it
    e = hipMemset(p, 0, SC_STATIC_SCRATCH_BYTES);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(e, "hipMemset (static scratch)");
    g_scratch[dev] = static_cast<uint8_t*>(p);
  }
  *out = g_scratch[dev];
  return SC_OK;
}

}  // namespace

struct sc_handle {
  sc_config cfg;
  std::vector<int32_t> S;
  Shape sh;
  int Pmax;
  int ev_cap;
  uint8_t* d_pool;
  uint8_t* d_state;
  uint8_t* d_ws;
  std::vector<size_t> pool_off;     // per layer, in d_pool
  std::vector<size_t> state_off;    // per layer, in d_state
  std::vector<LayerOffsets> lo;
  size_t gs_off;                    // banks' gs tables in d_state
  WsOffsets wo;
  Workspace W;
  std::vector<void*> bank_host;
  std::vector<void*> bank_dev;
  hipStream_t last_stream;
  bool stepped;
  std::vector<std::vector<int32_t>> pins;   // per layer: experts pinned in slots 0..P-1
  bool timed;                       // the last step was a timed one (spans written)
  uint64_t* d_span;                 // [SC_N_KERNELS][span_cap][kSpanSlots]
  int span_cap;
  int clock_khz;                    // wall clock rate of the span stamps
  Workspace last_W;                 // workspace of the last step (read_routing reads it)
  int device;                       // device the handle was set up on
  bool static_ok;                   // moe_layer_decode_static can run (scratch found and large enough)
  size_t static_need;               // bytes of static scratch the configuration needs
  std::string static_err;           // why it cannot, otherwise
  Workspace W_static;               // the static scratch laid out for this configuration
};

namespace {

struct Sizes {
  size_t pool, state, ws, bank;
  std::vector<size_t> pool_off, state_off;
  std::vector<LayerOffsets> lo;
  size_t gs_off;
  WsOffsets wo;
};

Sizes compute_sizes(const sc_config* c) {
  Sizes z;
  Shape sh = make_shape(c->hidden, c->inter, c->n_experts, c->top_k);
  int cap = ev_cap_of(c);
  size_t pool = 0, state = 0;
  for (int l = 0; l < c->n_layers; ++l) {
    z.pool_off.push_back(pool);
    pool += align_up((size_t)c->slots_per_layer[l] * (size_t)sh.blob);
    LayerOffsets o = layer_offsets(c->n_experts, c->slots_per_layer[l], cap);
    z.lo.push_back(o);
    z.state_off.push_back(state);
    state += o.end;
  }
  z.gs_off = state;
  state += align_up((size_t)c->n_banks * c->n_experts * 2 * sizeof(float));
  z.pool = pool;
  z.state = state;
  z.wo = ws_offsets(c->max_rows * c->top_k, c->hidden, c->inter, c->max_rows, stage_experts(c), sh.blob);
  z.ws = z.wo.end;
  z.bank = (size_t)c->n_experts * (size_t)sh.blob;
  return z;
}

LayerDev layer_dev(sc_handle* h, int l) {
  LayerDev L;
  uint8_t* base = h->d_state + h->state_off[l];
  const LayerOffsets& o = h->lo[l];
  L.e2s = reinterpret_cast<int32_t*>(base + o.e2s);
  L.s2e = reinterpret_cast<int32_t*>(base + o.s2e);
  L.key = reinterpret_cast<int64_t*>(base + o.key);
  L.step = reinterpret_cast<int64_t*>(base + o.misc + kMiscStep);
  L.counters = reinterpret_cast<uint64_t*>(base + o.misc + kMiscCounters);
  L.ev_head = reinterpret_cast<uint64_t*>(base + o.misc + kMiscEvHead);
  L.error = reinterpret_cast<uint32_t*>(base + o.misc + kMiscError);
  L.events = reinterpret_cast<sc_event*>(base + o.events);
  L.slots = h->d_pool + h->pool_off[l];
  const int bank = l % h->cfg.n_banks;
  L.backing = static_cast<const uint8_t*>(h->bank_dev[bank]);
  L.gs = reinterpret_cast<const float*>(h->d_state + h->gs_off) + (size_t)bank * h->sh.E * 2;
  L.S = h->S[l];
  L.ev_cap = h->ev_cap;
  L.P = (int32_t)h->pins[l].size();
  return L;
}

sc_status sync_last(sc_handle* h) {
  hipError_t e = h->stepped ? hipStreamSynchronize(h->last_stream) : hipSuccess;
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  return SC_OK;
}

sc_status check_layer(sc_handle* h, int layer) {
  if (!h) return fail(SC_E_ARG, "handle is NULL");
  if (layer < 0 || layer >= h->cfg.n_layers) return fail(SC_E_ARG, "layer %d out of range", layer);
  return SC_OK;
}

// Writes a layer's maps, keys and step counter from host images.
sc_status put_state(sc_handle* h, int l, const std::vector<int32_t>& e2s, const std::vector<int32_t>& s2e,
                    const std::vector<int64_t>& key, int64_t step) {
  LayerDev L = layer_dev(h, l);
  hipError_t e;
  if ((e = hipMemcpy(L.e2s, e2s.data(), e2s.size() * 4, hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipMemcpy(L.s2e, s2e.data(), s2e.size() * 4, hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipMemcpy(L.key, key.data(), key.size() * 8, hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipMemcpy(L.step, &step, 8, hipMemcpyHostToDevice)) != hipSuccess)
    return hip_fail(e, "hipMemcpy (state)");
  return SC_OK;
}

}  // namespace

extern "C" {

sc_status slotcache_query_sizes(const sc_config* cfg, sc_sizes* out) {
  sc_status st = check_config(cfg);
  if (st != SC_OK) return st;
  if (!out) return fail(SC_E_ARG, "out is NULL");
  Sizes z = compute_sizes(cfg);
  out->blob_bytes = (size_t)make_shape(cfg->hidden, cfg->inter, cfg->n_experts, cfg->top_k).blob;
  out->slot_pool_bytes = z.pool;
  out->state_bytes = z.state;
  out->workspace_bytes = z.ws;
  out->backing_bytes_per_bank = z.bank;
  return SC_OK;
}

sc_status slotcache_init(const sc_config* cfg, void* d_slot_pool, void* d_state, void* d_workspace,
                         sc_handle** out) {
  sc_status st = check_config(cfg);
  if (st != SC_OK) return st;
  if (!out) return fail(SC_E_ARG, "out is NULL");
  *out = nullptr;
  if (!d_slot_pool || !d_state || !d_workspace) return fail(SC_E_ARG, "device buffer is NULL");
  if (((uintptr_t)d_slot_pool | (uintptr_t)d_state | (uintptr_t)d_workspace) % kAlign)
    return fail(SC_E_ARG, "device buffers must be %zu-byte aligned", kAlign);
  Sizes z = compute_sizes(cfg);
  sc_handle* h = new sc_handle();
  h->cfg = *cfg;
  h->S.assign(cfg->slots_per_layer, cfg->slots_per_layer + cfg->n_layers);
  h->cfg.slots_per_layer = h->S.data();
  h->sh = make_shape(cfg->hidden, cfg->inter, cfg->n_experts, cfg->top_k);
  h->Pmax = cfg->max_rows * cfg->top_k;
  h->ev_cap = ev_cap_of(cfg);
  h->d_pool = static_cast<uint8_t*>(d_slot_pool);
  h->d_state = static_cast<uint8_t*>(d_state);
  h->d_ws = static_cast<uint8_t*>(d_workspace);
  h->pool_off = z.pool_off;
  h->state_off = z.state_off;
  h->lo = z.lo;
  h->gs_off = z.gs_off;
  h->wo = z.wo;
  h->last_stream = nullptr;
  h->stepped = false;
  h->pins.assign(cfg->n_layers, {});
  for (int b = 0; b < cfg->n_banks; ++b) {
    void* p = nullptr;
    hipError_t e = hipHostMalloc(&p, z.bank, hipHostMallocDefault);
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      slotcache_destroy(h);
      return fail(SC_E_HOST_OOM, "hipHostMalloc of %zu bytes for bank %d failed", z.bank, b);
    }
    h->bank_host.push_back(p);
    void* d = nullptr;
    e = hipHostGetDevicePointer(&d, p, 0);
    if (e != hipSuccess || !d) {
      slotcache_destroy(h);
      return hip_fail(e, "hipHostGetDevicePointer");
    }
    h->bank_dev.push_back(d);
  }
  const WsOffsets& o = h->wo;
  h->W = bind_workspace(h->d_ws, o, stage_experts(cfg));
  h->last_W = h->W;
  h->d_span = reinterpret_cast<uint64_t*>(h->d_ws + o.span);
  h->span_cap = span_blocks(cfg->max_rows, cfg->hidden);
  h->timed = false;
  h->clock_khz = 0;
  h->device = 0;
  if (hipGetDevice(&h->device) != hipSuccess ||
      hipDeviceGetAttribute(&h->clock_khz, hipDeviceAttributeWallClockRate, h->device) != hipSuccess)
    (void)hipGetLastError();
  // the static scratch of this device (moe_layer_decode_static); a failure here
  // only disables that entry point, which then reports it
  {
    const WsOffsets so = static_offsets(cfg);
    h->static_need = so.end;
    h->static_ok = false;
    uint8_t* base = nullptr;
    if (so.end > (size_t)SC_STATIC_SCRATCH_BYTES) {
      char buf[160];
      snprintf(buf, sizeof buf, "the configuration needs %zu bytes of per-call scratch, the static array holds %zu",
               so.end, (size_t)SC_STATIC_SCRATCH_BYTES);
      h->static_err = buf;
    } else if (static_scratch(h->device, &base) != SC_OK) {
      h->static_err = g_err;
    } else {
      h->W_static = bind_workspace(base, so, 0);
      h->static_ok = true;
    }
  }

  // Cold state: every slot empty, keys -1, counters and rings zero, gs = 1.
  std::vector<uint8_t> img(z.state, 0);
  for (int l = 0; l < cfg->n_layers; ++l) {
    uint8_t* base = img.data() + z.state_off[l];
    const LayerOffsets& lo = z.lo[l];
    int32_t* e2s = reinterpret_cast<int32_t*>(base + lo.e2s);
    int32_t* s2e = reinterpret_cast<int32_t*>(base + lo.s2e);
    int64_t* key = reinterpret_cast<int64_t*>(base + lo.key);
    for (int e = 0; e < cfg->n_experts; ++e) e2s[e] = -1;
    for (int s = 0; s < h->S[l]; ++s) {
      s2e[s] = -1;
      key[s] = -1;
    }
  }
  float* gs = reinterpret_cast<float*>(img.data() + z.gs_off);
  for (size_t i = 0; i < (size_t)cfg->n_banks * cfg->n_experts * 2; ++i) gs[i] = 1.0f;
  hipError_t e = hipMemcpy(h->d_state, img.data(), z.state, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemset(h->d_ws, 0, z.ws);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    slotcache_destroy(h);
    return hip_fail(e, "state initialisation");
  }
  *out = h;
  return SC_OK;
}

sc_status slotcache_backing(sc_handle* h, int32_t bank, void** host_ptr, size_t* bytes) {
  if (!h) return fail(SC_E_ARG, "handle is NULL");
  if (bank < 0 || bank >= h->cfg.n_banks) return fail(SC_E_ARG, "bank %d out of range", bank);
  if (host_ptr) *host_ptr = h->bank_host[bank];
  if (bytes) *bytes = (size_t)h->sh.E * (size_t)h->sh.blob;
  return SC_OK;
}

sc_status slotcache_set_global_scales(sc_handle* h, int32_t bank, const float* h_gs) {
  if (!h) return fail(SC_E_ARG, "handle is NULL");
  if (bank < 0 || bank >= h->cfg.n_banks) return fail(SC_E_ARG, "bank %d out of range", bank);
  if (!h_gs) return fail(SC_E_ARG, "gs is NULL");
  sc_status st = sync_last(h);
  if (st != SC_OK) return st;
  float* d = reinterpret_cast<float*>(h->d_state + h->gs_off) + (size_t)bank * h->sh.E * 2;
  hipError_t e = hipMemcpy(d, h_gs, (size_t)h->sh.E * 2 * sizeof(float), hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy (global scales)");
  return SC_OK;
}

sc_status slotcache_preload(sc_handle* h, int32_t layer) {
  sc_status st = check_layer(h, layer);
  if (st != SC_OK) return st;
  if ((st = sync_last(h)) != SC_OK) return st;
  const int S = h->S[layer];
  LayerDev L = layer_dev(h, layer);
  hipError_t e = hipMemcpy(L.slots, L.backing, (size_t)S * (size_t)h->sh.blob, hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy (preload)");
  std::vector<int32_t> e2s(h->sh.E, -1), s2e(S);
  std::vector<int64_t> key(S, -1);
  for (int s = 0; s < S; ++s) {
    e2s[s] = s;
    s2e[s] = s;
  }
  int64_t step = 0;
  e = hipMemcpy(&step, L.step, 8, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy (step)");
  h->pins[layer].clear();
  return put_state(h, layer, e2s, s2e, key, step);
}

sc_status slotcache_pin(sc_handle* h, int32_t layer, const int32_t* h_experts, int32_t n) {
  sc_status st = check_layer(h, layer);
  if (st != SC_OK) return st;
  const int S = h->S[layer], E = h->sh.E;
  if (n < 0 || n > S) return fail(SC_E_ARG, "n=%d must be in [0, S=%d]", n, S);
  if (n > 0 && !h_experts) return fail(SC_E_ARG, "experts is NULL");
  std::vector<int32_t> pins(h_experts, h_experts + n);
  std::vector<char> seen(E, 0);
  for (int i = 0; i < n; ++i) {
    if (pins[i] < 0 || pins[i] >= E) return fail(SC_E_ARG, "expert %d out of range", pins[i]);
    if (seen[pins[i]]) return fail(SC_E_ARG, "expert %d pinned twice", pins[i]);
    seen[pins[i]] = 1;
  }
  if ((st = sync_last(h)) != SC_OK) return st;
  LayerDev L = layer_dev(h, layer);
  for (int i = 0; i < n; ++i) {
    hipError_t e = hipMemcpy(L.slots + (size_t)i * h->sh.blob, L.backing + (size_t)pins[i] * h->sh.blob,
                             (size_t)h->sh.blob, hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy (pin)");
  }
  std::vector<int32_t> e2s(E, -1), s2e(S, -1);
  std::vector<int64_t> key(S, -1);
  for (int i = 0; i < n; ++i) {
    s2e[i] = pins[i];
    e2s[pins[i]] = i;
  }
  int64_t step = 0;
  hipError_t e = hipMemcpy(&step, L.step, 8, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy (step)");
  if ((st = put_state(h, layer, e2s, s2e, key, step)) != SC_OK) return st;
  h->pins[layer] = pins;
  return SC_OK;
}

namespace {

sc_status check_step(sc_handle* h, int32_t layer, const float* d_logits, const uint16_t* d_x, int32_t M,
                     float* d_y) {
  sc_status st = check_layer(h, layer);
  if (st != SC_OK) return st;
  if (M < 1 || M > h->cfg.max_rows) return fail(SC_E_ARG, "M=%d must be in [1, %d]", M, h->cfg.max_rows);
  if (!d_logits || !d_x || !d_y) return fail(SC_E_ARG, "logits, x and y must be non-NULL");
  return SC_OK;
}

// Enqueues one step whose per-call scratch is `W` (arguments already checked).
sc_status enqueue_step(sc_handle* h, int32_t layer, const float* d_logits, const uint16_t* d_x, int32_t M,
                       float* d_y, void* stream, void* const* events, const Workspace& W) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  LayerDev L = layer_dev(h, layer);
  hipError_t e = hipSuccess;
  auto kev = [&](int i) {
    KEvents k;
    if (events) {
      k.start = static_cast<hipEvent_t>(events[2 * i]);
      k.stop = static_cast<hipEvent_t>(events[2 * i + 1]);
      k.span = h->d_span + (size_t)i * h->span_cap * kSpanSlots;
      k.span_blocks = h->span_cap;
    }
    return k;
  };
  const bool mfma = !(h->cfg.flags & SC_FLAG_BATCH_INVARIANT);
  e = launch_route(h->sh, L, W, d_logits, M, s, kev(0));
  if (M == 1 && (h->cfg.flags & SC_FLAG_OVERLAP_FILL)) {
    // the copy shares a launch with the resident experts' gate/up; the copied
    // experts' gate/up runs after it
    KEvents fev = kev(1);
    if (e == hipSuccess && fev.start) e = hipEventRecord(fev.start, s);
    if (e == hipSuccess) e = launch_fill_gateup(h->sh, W, L.gs, d_x, s, fev, kev(2));
    if (e == hipSuccess && fev.stop) e = hipEventRecord(fev.stop, s);
    if (e == hipSuccess) e = launch_gateup_filled(h->sh, W, L.gs, d_x, s);
    if (e == hipSuccess) e = launch_down(h->sh, W, L.gs, M, mfma, -1, s, kev(3));
  } else if (!staged_step(W, M)) {
    if (e == hipSuccess) e = launch_fill(h->sh, W, -1, s, kev(1));
    if (e == hipSuccess) e = launch_gateup(h->sh, W, L.gs, d_x, M, mfma, -1, s, kev(2));
    if (e == hipSuccess) e = launch_down(h->sh, W, L.gs, M, mfma, -1, s, kev(3));
  } else {
    // prefill groups: copy G experts into staging, compute them, next group
    const int ng = stage_groups(W, M, h->sh.k, h->sh.E);
    for (int g = 0; g < ng && e == hipSuccess; ++g) {
      auto gev = [&](int i) { return g == 0 ? kev(i) : KEvents(); };
      e = launch_fill(h->sh, W, g, s, gev(1));
      if (e == hipSuccess) e = launch_gateup(h->sh, W, L.gs, d_x, M, mfma, g, s, gev(2));
      if (e == hipSuccess) e = launch_down(h->sh, W, L.gs, M, mfma, g, s, gev(3));
    }
  }
  if (e == hipSuccess) e = launch_combine(h->sh, W, d_y, M, s, kev(4));
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  h->last_stream = s;
  h->stepped = true;
  h->timed = events != nullptr;
  h->last_W = W;
  return SC_OK;
}

}  // namespace

sc_status moe_layer_decode_ev(sc_handle* h, int32_t layer, const float* d_logits, const uint16_t* d_x,
                              int32_t M, float* d_y, void* stream, void* const* events) {
  sc_status st = check_step(h, layer, d_logits, d_x, M, d_y);
  if (st != SC_OK) return st;
  return enqueue_step(h, layer, d_logits, d_x, M, d_y, stream, events, h->W);
}

sc_status moe_layer_decode(sc_handle* h, int32_t layer, const float* d_logits, const uint16_t* d_x,
                           int32_t M, float* d_y, void* stream) {
  return moe_layer_decode_ev(h, layer, d_logits, d_x, M, d_y, stream, nullptr);
}

sc_status moe_layer_decode_static(sc_handle* h, int32_t layer, const float* d_logits, const uint16_t* d_x,
                                  int32_t M, float* d_y, void* stream) {
  sc_status st = check_step(h, layer, d_logits, d_x, M, d_y);
  if (st != SC_OK) return st;
  if (M > kCachedRows)
    return fail(SC_E_ARG, "M=%d: moe_layer_decode_static takes at most %d rows (prefill chunks stage through the "
                "caller's workspace)", M, kCachedRows);
  if (!h->static_ok) return fail(SC_E_ARG, "moe_layer_decode_static: %s", h->static_err.c_str());
  return enqueue_step(h, layer, d_logits, d_x, M, d_y, stream, nullptr, h->W_static);
}

sc_status slotcache_read_kernel_spans(sc_handle* h, double* us_out) {
  if (!h) return fail(SC_E_ARG, "handle is NULL");
  if (!us_out) return fail(SC_E_ARG, "us_out is NULL");
  if (!h->timed) return fail(SC_E_STATE, "the last step was not run through moe_layer_decode_ev");
  if (h->clock_khz <= 0) return fail(SC_E_UNSUPPORTED, "device wall clock rate unknown");
  sc_status st = sync_last(h);
  if (st != SC_OK) return st;
  const size_t per = (size_t)h->span_cap * kSpanSlots;
  std::vector<uint64_t> s((size_t)SC_N_KERNELS * per);
  hipError_t e = hipMemcpy(s.data(), h->d_span, s.size() * 8, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy (spans)");
  // stamps older than this step's routing kernel start are left over from earlier steps
  const uint64_t t0 = s[0];
  for (int i = 0; i < SC_N_KERNELS; ++i) {
    uint64_t lo = UINT64_MAX, hi = 0;
    for (int b = 0; b < h->span_cap; ++b) {
      const uint64_t* r = &s[i * per + (size_t)b * kSpanSlots];
      if (r[0] >= t0 && r[0] < lo) lo = r[0];
      for (int w = 1; w < kSpanSlots; ++w)
        if (r[w] >= t0 && r[w] > hi) hi = r[w];
    }
    us_out[i] = (lo == UINT64_MAX || hi < lo) ? 0.0 : (double)(hi - lo) * 1000.0 / (double)h->clock_khz;
  }
  return SC_OK;
}

sc_status slotcache_stats(sc_handle* h, int32_t layer, sc_stats* out) {
  sc_status st = check_layer(h, layer);
  if (st != SC_OK) return st;
  if (!out) return fail(SC_E_ARG, "out is NULL");
  if ((st = sync_last(h)) != SC_OK) return st;
  LayerDev L = layer_dev(h, layer);
  uint64_t c[C_N];
  uint32_t err = 0;
  hipError_t e = hipMemcpy(c, L.counters, sizeof c, hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemcpy(&err, L.error, 4, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy (stats)");
  out->steps = c[C_STEPS];
  out->bypass_steps = c[C_BYPASS];
  out->picks = c[C_PICKS];
  out->lookups = c[C_LOOKUPS];
  out->hits = c[C_HITS];
  out->misses = c[C_MISSES];
  out->evictions = c[C_EVICT];
  out->bytes_filled = c[C_FILLED];
  out->bypass_bytes = c[C_BYPASS_BYTES];
  out->device_error = err;
  out->reserved = 0;
  if (err) return fail(SC_E_DEVICE, "device error word 0x%x on layer %d", err, layer);
  return SC_OK;
}

sc_status slotcache_read_state(sc_handle* h, int32_t layer, int32_t* h_e2s, int32_t* h_s2e, int64_t* h_key,
                               int64_t* h_step) {
  sc_status st = check_layer(h, layer);
  if (st != SC_OK) return st;
  if ((st = sync_last(h)) != SC_OK) return st;
  LayerDev L = layer_dev(h, layer);
  const int S = h->S[layer];
  hipError_t e = hipSuccess;
  if (h_e2s && e == hipSuccess) e = hipMemcpy(h_e2s, L.e2s, (size_t)h->sh.E * 4, hipMemcpyDeviceToHost);
  if (h_s2e && e == hipSuccess) e = hipMemcpy(h_s2e, L.s2e, (size_t)S * 4, hipMemcpyDeviceToHost);
  if (h_key && e == hipSuccess) e = hipMemcpy(h_key, L.key, (size_t)S * 8, hipMemcpyDeviceToHost);
  if (h_step && e == hipSuccess) e = hipMemcpy(h_step, L.step, 8, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy (read_state)");
  return SC_OK;
}

sc_status slotcache_write_state(sc_handle* h, int32_t layer, const int32_t* h_e2s, const int32_t* h_s2e,
                                const int64_t* h_key, int64_t step) {
  sc_status st = check_layer(h, layer);
  if (st != SC_OK) return st;
  if (!h_e2s || !h_s2e || !h_key) return fail(SC_E_ARG, "state arrays must be non-NULL");
  // the remap packs (key + 2) above an 11-bit slot index in 64 bits and stamps
  // keys t * 16k + position: a step below 2^40 keeps both far from overflow
  if (step < 0 || step >= kMaxStateStep) return fail(SC_E_ARG, "step must be in [0, 2^40)");
  const int E = h->sh.E, S = h->S[layer];
  // a key the layer could have stamped: -1 (filled, never referenced since) or
  // t * 16k + position for some earlier step t
  const int64_t key_end = step * (int64_t)(kCachedRows * h->sh.k);
  for (int e = 0; e < E; ++e) {
    int s = h_e2s[e];
    if (s < -1 || s >= S || (s >= 0 && h_s2e[s] != e))
      return fail(SC_E_ARG, "e2s[%d]=%d is not the inverse of s2e", e, s);
  }
  for (int s = 0; s < S; ++s) {
    int e = h_s2e[s];
    if (e < -1 || e >= E || (e >= 0 && h_e2s[e] != s))
      return fail(SC_E_ARG, "s2e[%d]=%d is not the inverse of e2s", s, e);
    if (e < 0 && h_key[s] != -1) return fail(SC_E_ARG, "empty slot %d must have key -1", s);
    if (e >= 0 && (h_key[s] < -1 || h_key[s] >= key_end))
      return fail(SC_E_ARG, "key[%d]=%lld of an occupied slot must be in [-1, step*16*k = %lld)", s,
                  (long long)h_key[s], (long long)key_end);
  }
  const std::vector<int32_t>& pins = h->pins[layer];
  for (size_t s = 0; s < pins.size(); ++s)
    if (h_s2e[s] != pins[s]) return fail(SC_E_ARG, "pinned slot %zu must keep expert %d", s, pins[s]);
  if ((st = sync_last(h)) != SC_OK) return st;
  LayerDev L = layer_dev(h, layer);
  for (int s = 0; s < S; ++s) {
    int e = h_s2e[s];
    if (e < 0) continue;
    hipError_t err = hipMemcpy(L.slots + (size_t)s * h->sh.blob, L.backing + (size_t)e * h->sh.blob,
                               (size_t)h->sh.blob, hipMemcpyHostToDevice);
    if (err != hipSuccess) return hip_fail(err, "hipMemcpy (refill)");
  }
  return put_state(h, layer, std::vector<int32_t>(h_e2s, h_e2s + E), std::vector<int32_t>(h_s2e, h_s2e + S),
                   std::vector<int64_t>(h_key, h_key + S), step);
}

sc_status slotcache_read_events(sc_handle* h, int32_t layer, sc_event* h_buf, size_t cap, size_t* n_out,
                                uint64_t* total) {
  sc_status st = check_layer(h, layer);
  if (st != SC_OK) return st;
  if ((st = sync_last(h)) != SC_OK) return st;
  LayerDev L = layer_dev(h, layer);
  uint64_t head = 0;
  hipError_t e = hipMemcpy(&head, L.ev_head, 8, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy (ev_head)");
  const uint64_t ring = (uint64_t)h->ev_cap;
  uint64_t avail = head < ring ? head : ring;
  uint64_t n = avail < (uint64_t)cap ? avail : (uint64_t)cap;
  if (n > 0 && !h_buf) return fail(SC_E_ARG, "buffer is NULL");
  std::vector<sc_event> all(ring);
  if (n > 0) {
    e = hipMemcpy(all.data(), L.events, ring * sizeof(sc_event), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy (events)");
    const uint64_t first = head - avail;     // oldest still in the ring
    for (uint64_t i = 0; i < n; ++i) h_buf[i] = all[(first + i) % ring];
  }
  if (n_out) *n_out = (size_t)n;
  if (total) *total = head;
  return SC_OK;
}

sc_status slotcache_read_routing(sc_handle* h, int32_t* h_ids, float* h_w, int32_t* M_out, int32_t* bypass) {
  if (!h) return fail(SC_E_ARG, "handle is NULL");
  if (!h->stepped) return fail(SC_E_STATE, "no step has run on this handle");
  sc_status st = sync_last(h);
  if (st != SC_OK) return st;
  int32_t hdr[H_WORDS];
  const Workspace& W = h->last_W;
  hipError_t e = hipMemcpy(hdr, W.hdr, sizeof hdr, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy (hdr)");
  const int M = hdr[H_ROWS], P = M * h->sh.k;
  if (h_ids && e == hipSuccess) e = hipMemcpy(h_ids, W.pick_expert, (size_t)P * 4, hipMemcpyDeviceToHost);
  if (h_w && e == hipSuccess) e = hipMemcpy(h_w, W.pick_w, (size_t)P * 4, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy (routing)");
  if (M_out) *M_out = M;
  if (bypass) *bypass = hdr[H_BYPASS];
  return SC_OK;
}

const char* slotcache_last_error(void) { return g_err.c_str(); }

void slotcache_destroy(sc_handle* h) {
  if (!h) return;
  (void)hipDeviceSynchronize();
  for (void* p : h->bank_host)
    if (p) (void)hipHostFree(p);
  delete h;
}

}  // extern "C"
