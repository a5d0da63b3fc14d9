/*
 * slotcache.h -- C ABI of the expert-slot MoE decode step for MI355X (gfx950).
 *
 * One MoE layer of an expert-offloaded mixture-of-experts model keeps S fixed
 * HBM slots, each able to hold one routed expert; every expert of the layer
 * lives in a pinned host backing store, and the slots are an LRU cache over
 * it.  One decode step (moe_layer_decode) runs, all on the device and all
 * enqueued on the caller's stream:
 *   router top-k -> expert id to slot remap with LRU victim choice -> copy of
 *   missed experts' weight and scale rows from host into their victim slots ->
 *   routed gate/up and down products on NVFP4 weights with SiLU -> weighted
 *   top-k combine.
 * The method is the slot cache of the page "GLM 5.3 Testing: HBM Expert
 * Allocation" (sections "What the slot cache is" and "The build, measured on a
 * synthetic GLM-shaped layer"), with the LRU occupancy of the page "GB300 GLM
 * 5.3 Testing" (section "Expert allocation vs a cache").
 *
 * Conventions.
 *  - Every call returns sc_status: SC_OK (0) or a negative error; nothing
 *    aborts or throws.  slotcache_last_error() gives a message for the last
 *    non-OK status on the calling thread.
 *  - Pointers named d_* are device pointers (hipMalloc / torch CUDA tensors);
 *    pointers named h_* or host_* are host pointers.  `stream` is a
 *    hipStream_t passed as void* (NULL = the null stream).
 *  - The caller owns every device buffer (slot pool, state, workspace,
 *    logits, x, y) and the stream.  The library owns the pinned host backing
 *    store (allocated at the exact size, no power-of-two rounding) and frees
 *    it in slotcache_destroy.
 *  - Calls that use one handle must be ordered: the same stream, or streams
 *    the caller synchronizes.  They share one workspace.
 *
 * Data formats (one expert "blob", B_e bytes; the same layout in a slot and in
 * the backing store):
 *   [w13 codes  2I x H/2 bytes] rows 0..I-1 gate, rows I..2I-1 up
 *   [w13 scales 2I x H/16     ] one FP8 E4M3 (OCP "FN") per 16 K-elements
 *   [w2 codes   H x I/2       ]
 *   [w2 scales  H x I/16      ]
 *   Codes are FP4 E2M1, two per byte, the even element in the low nibble.
 *   Element value = e2m1(code) * e4m3(block scale) * global scale, with one
 *   fp32 global scale per (expert, matrix) held in a device table.
 *   B_e = 27*H*I/16 (21,233,664 B for H=6144, I=2048).
 */
#ifndef SLOTCACHE_H
#define SLOTCACHE_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define SC_API __attribute__((visibility("default")))
#else
#define SC_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SC_OK = 0,
  SC_E_ARG = -1,          /* invalid argument or configuration; nothing enqueued */
  SC_E_HOST_OOM = -2,     /* pinned host allocation failed */
  SC_E_HIP = -3,          /* a HIP runtime call failed */
  SC_E_STATE = -4,        /* call not valid in the handle's state */
  SC_E_DEVICE = -5,       /* a device-side check latched an error word */
  SC_E_UNSUPPORTED = -6   /* shape outside the compiled kernel set */
} sc_status;

typedef struct sc_handle sc_handle;

/* Rows per step above which a step always reads the backing store directly
 * (the prefill bypass; page "GLM 5.3 Testing: HBM Expert Allocation", section
 * "What the slot cache is"). */
#define SC_BYPASS_ROWS 16

typedef struct {
  int32_t n_layers;               /* >= 1 */
  int32_t hidden;                 /* H: 256, 512, 1024, 2048, 4096, 6144 or 8192 */
  int32_t inter;                  /* I: 128 ... 8192 (same set plus 128) */
  int32_t n_experts;              /* E: top_k <= E <= 1024 */
  int32_t top_k;                  /* k: 1 <= k <= 32 */
  const int32_t* slots_per_layer; /* host [n_layers]; 1 <= S_l <= min(E, 1024) */
  int32_t max_rows;               /* largest M the caller will pass, 1..256 */
  int32_t n_banks;                /* host backing banks, 1..n_layers; layer l reads bank l % n_banks */
  int32_t event_capacity;         /* per-layer miss-event ring, records (0 = 4096) */
  uint32_t flags;                 /* 0, or SC_FLAG_BATCH_INVARIANT and/or SC_FLAG_OVERLAP_FILL */
  int32_t prefill_stage;          /* G, experts staged per prefill group, 0..1024 (see below) */
} sc_config;

/* Prefill groups.  A step of more than SC_BYPASS_ROWS rows (a prefill chunk)
 * always bypasses the cache.  With prefill_stage = 0 its non-resident experts
 * are read in place from the host-mapped backing store by the expert kernels.
 * With G = prefill_stage > 0 the workspace holds a G-blob staging area in HBM:
 * the step's non-resident experts, in first-occurrence order, are copied into
 * it G at a time by the fill kernel, and each group's expert products (the
 * resident experts go with the first group) run from HBM before the next
 * group is copied; the weighted combine runs once, after the last group, so
 * the output is the same bits as without staging.  The pages' prefill-groups
 * knob stages 64 experts at a time and reduces once (page "glm53 -
 * GLM-5.3-Flash (NVFP4)").  A step of M rows enqueues ceil(min(M*k, E) / G)
 * groups; groups left empty exit at once.  Ignored (no staging area) when
 * max_rows <= SC_BYPASS_ROWS. */

/* Every row of a step computes the bits it would compute alone, as a one-row
 * step: the streaming FP4 kernels run for every M (their per-row reduction
 * order does not depend on how many rows share an expert) and the matrix-core
 * kernels, whose rounding differs, are not used.  Drafted and verify rows then
 * never change a row's output (the exact-decoding rule on the page "TensorFold
 * GLM-5.3 explained").  Costs speed from M = 5 on (the matrix-core ranges
 * below). */
#define SC_FLAG_BATCH_INVARIANT 1u

/* Overlapped miss fill for one-row steps (M = 1).  The copy of the step's
 * misses into their slots shares one launch with the gate/up products of the
 * experts it does not write, which run while the copy crosses the host link;
 * the copied experts' gate/up follows, then down and the combine.  The pages
 * name asynchronous miss fills as what could take the copy off the critical
 * path (page "GB300 GLM 5.3 Testing", September 13 update of the section
 * "Speculation: what is holding the GB300 back, and what probably wins
 * next").  Outputs, slots and bookkeeping are the same bits as without the
 * flag.  The trade-off: a step with misses finishes sooner by about the
 * resident experts' gate/up time, but the copy blocks take wave slots from
 * the products, so an all-hit step's gate/up runs slower.  Steps of more than
 * one row are not affected.  With events (moe_layer_decode_ev) both the
 * fill and the gate/up events bracket the shared launch; the fill spans are
 * those of its copy blocks and the gate/up spans those of its product blocks
 * (slotcache_read_kernel_spans); the copied experts' gate/up launch is not
 * timed. */
#define SC_FLAG_OVERLAP_FILL 2u

/* Without SC_FLAG_BATCH_INVARIANT, steps of at least this many rows run the
 * gate/up (resp. down) product on the matrix cores; their rows need not be
 * bit-equal to the same rows decoded alone (the outputs stay within the same
 * tolerance of the exact result).  Below them the streaming kernels run, whose
 * rows are bit-equal to one-row steps: on steps of 2 to 4 rows both products
 * keep the expert's pick operands in LDS and widen each weight once for all
 * of them. */
#define SC_MFMA_MIN_ROWS_GATEUP 5
#define SC_MFMA_MIN_ROWS_DOWN 5

typedef struct {
  size_t blob_bytes;              /* B_e */
  size_t slot_pool_bytes;         /* device: sum over layers of S_l * B_e; 256-B aligned base */
  size_t state_bytes;             /* device: maps, LRU keys, counters, event rings, global scales */
  size_t workspace_bytes;         /* device: per-call scratch shared by all layers, with the
                                     prefill staging area (G * B_e) when there is one */
  size_t backing_bytes_per_bank;  /* host, allocated by the library: E * B_e */
} sc_sizes;

typedef struct {
  uint64_t steps;         /* calls of moe_layer_decode on the layer */
  uint64_t bypass_steps;  /* steps that read the backing store directly */
  uint64_t picks;         /* M*k over cached steps */
  uint64_t lookups;       /* unique experts over cached steps */
  uint64_t hits;          /* unique experts already resident */
  uint64_t misses;        /* unique experts copied into a slot */
  uint64_t evictions;     /* misses whose victim slot held an expert */
  uint64_t bytes_filled;  /* misses * B_e, host to HBM */
  uint64_t bypass_bytes;  /* unique experts * B_e read from host by bypass steps */
  uint32_t device_error;  /* nonzero: a device-side bounds check failed */
  uint32_t reserved;
} sc_stats;

typedef struct {
  int64_t step;     /* value of the layer's step counter when the miss happened */
  int32_t expert;   /* expert copied in */
  int32_t slot;     /* its slot */
  int32_t evicted;  /* expert that held the slot, or -1 for an empty slot */
  int32_t reserved;
} sc_event;

/* Sizes of the device buffers the caller must allocate for `cfg`, so that every
 * device buffer is sized once, up front, before any step runs.  The pages lost
 * launches to memory that was taken after the budget had been set (page "glm53 -
 * GLM-5.3-Flash (NVFP4)", section "Context and the KV cap": a cache allocated
 * after the framework's memory profiling) and to budgets checked in the wrong
 * units (page "GLM 5.3 Testing: HBM Expert Allocation", section "Five launches,
 * four failures").  Byte counts are exact (no rounding to a power of two).
 * Pure: no device or host allocation.  SC_E_ARG / SC_E_UNSUPPORTED for an
 * invalid or unsupported configuration; *out is left untouched then. */
SC_API sc_status slotcache_query_sizes(const sc_config* cfg, sc_sizes* out);

/* Binds caller-allocated device buffers (sizes from slotcache_query_sizes,
 * 256-byte aligned), allocates the pinned backing store (n_banks * E * B_e
 * bytes, exact size, device-mapped) and resets every layer to the cold state:
 * all slots empty, keys -1, counters zero, global scales 1.0.  Synchronous.
 * The device buffers must outlive the handle.
 * Page "GLM 5.3 Testing: HBM Expert Allocation": the per-layer slots and the
 * pinned backing store are section "What the slot cache is"; pinning at the
 * exact byte size (a rounding pinned allocator wasted a third of host memory)
 * is section "Five launches, four failures"; the cache starts empty and is
 * filled on demand (page "TensorFold GLM-5.3 explained": nothing is resident
 * for good).  Errors: SC_E_ARG (bad config, NULL or misaligned buffer),
 * SC_E_HOST_OOM (pinned allocation failed; nothing is kept), SC_E_HIP; *out is
 * NULL on any error. */
SC_API sc_status slotcache_init(const sc_config* cfg, void* d_slot_pool, void* d_state,
                         void* d_workspace, sc_handle** out);

/* Host pointer and size of backing bank `bank` ([E][B_e] blobs, expert-major).
 * The caller fills it before the first step that reads it and must not write
 * it while steps are in flight. */
SC_API sc_status slotcache_backing(sc_handle* h, int32_t bank, void** host_ptr, size_t* bytes);

/* Copies the fp32 global scales of bank `bank` from host memory h_gs[E][2]
 * ((w13, w2) per expert) to the device table.  Synchronous. */
SC_API sc_status slotcache_set_global_scales(sc_handle* h, int32_t bank, const float* h_gs);

/* Warm start for `layer`: slot s <- expert s for s < S (copied from the
 * backing store), keys -1, no pinned slots.  Synchronous.  With S == E this
 * makes every expert resident (the all-resident layer). */
SC_API sc_status slotcache_preload(sc_handle* h, int32_t layer);

/* One decode step of `layer` for M rows (1 <= M <= max_rows), the method of
 * page "GLM 5.3 Testing: HBM Expert Allocation", section "What the slot cache
 * is" (ids mapped to slots on the device before the expert launch, misses copied
 * into LRU victims, the expert products reading the same bytes as with every
 * expert resident, more than 16 rows bypassing, fixed addresses and shapes for
 * graph capture), with the fp32 combine of its section "A correction first":
 *   d_logits fp32 [M][E], d_x bf16 bits [M][H], d_y fp32 [M][H] (written).
 * Router: per row the k largest logits (ties -> lower expert id, NaN below
 * -inf), weights = softmax over the k chosen logits.  Cached steps (M <= 16
 * and at most S unique experts, see slotcache_pin for pinned slots) remap,
 * fill misses and compute from the slots; other steps (bypass) leave the cache
 * untouched and compute resident experts from their slots and the others from
 * the backing store.  Asynchronous on `stream`, no host synchronisation and no
 * allocation, so it can be captured into a HIP graph (fixed addresses and
 * shapes).  Argument errors return before anything is enqueued. */
SC_API sc_status moe_layer_decode(sc_handle* h, int32_t layer, const float* d_logits,
                           const uint16_t* d_x, int32_t M, float* d_y, void* stream);

/* Bytes of the library's static per-call scratch on each GPU (see
 * moe_layer_decode_static). */
#define SC_STATIC_SCRATCH_BYTES 16777216

/* moe_layer_decode for callers that cannot allocate: code under HIP graph
 * capture that must not touch an allocator, tight serving loops, harnesses
 * that forbid allocation.  The step's per-call scratch (routing lists, pick
 * grouping, h, per-pick down outputs) comes from a fixed device array of the
 * library, SC_STATIC_SCRATCH_BYTES per GPU, set up by slotcache_init on the
 * handle's device and held until the process ends, instead of the workspace
 * bound to the handle.  The caller still passes logits, x and y, and the
 * handle's slots and state are used as by moe_layer_decode; the results are
 * the same bits.  The call allocates nothing, host or device.
 * Every call on a GPU shares that GPU's array and leaves its contents behind
 * (each step writes every scratch word it reads before reading it, so nothing
 * needs clearing): calls that can overlap on one GPU -- streams not ordered
 * with each other, from this or any other handle -- race on it and must not
 * be issued.  slotcache_read_routing reads the array after such a step.
 * Errors (SC_E_ARG, nothing enqueued): the arguments of moe_layer_decode;
 * M > SC_BYPASS_ROWS (a prefill chunk needs the caller's workspace and its
 * staging area); a configuration whose per-call scratch for
 * min(max_rows, SC_BYPASS_ROWS) rows exceeds SC_STATIC_SCRATCH_BYTES (the
 * message gives both sizes); the array could not be set up at init. */
SC_API sc_status moe_layer_decode_static(sc_handle* h, int32_t layer, const float* d_logits,
                                         const uint16_t* d_x, int32_t M, float* d_y, void* stream);

/* Kernels of one step, for per-kernel timing: routing+remap, miss fill,
 * gate/up, down, combine. */
#define SC_N_KERNELS 5
#define SC_N_EVENTS (2 * SC_N_KERNELS)
/* moe_layer_decode with per-kernel timing: events[2i] and events[2i+1]
 * (hipEvent_t passed as void*, created by the caller) are stamped at the start
 * and the end of kernel i's execution (hipExtLaunchKernelGGL).  On a staged
 * prefill step the fill, gate/up and down events and spans are those of the
 * first group's launches.  events == NULL is moe_layer_decode. */
SC_API sc_status moe_layer_decode_ev(sc_handle* h, int32_t layer, const float* d_logits,
                              const uint16_t* d_x, int32_t M, float* d_y, void* stream,
                              void* const* events);

/* Pins experts of `layer` (hybrid policy: page "GB300 GLM 5.3 Testing",
 * section "Expert allocation vs a cache", compares a static pin with LRU):
 * slot i <- h_experts[i] for i < n (copied from the backing store), never a
 * victim; LRU runs over the other S - n slots, which are emptied (keys -1).
 * 0 <= n <= S distinct ids; n = 0 unpins.  The step counter and counters are
 * kept.  With n pinned slots a step bypasses when its unique experts outside
 * the pinned set exceed S - n (the rule |U| > S for n = 0); n = S is a static
 * pin.  slotcache_preload clears the pins; slotcache_write_state requires the
 * pinned slots to keep their experts.  Synchronous. */
SC_API sc_status slotcache_pin(sc_handle* h, int32_t layer, const int32_t* h_experts, int32_t n);

/* Execution spans of the kernels of the most recent step run through
 * moe_layer_decode_ev, in microseconds: us_out[i] (i < SC_N_KERNELS) is the
 * time from kernel i's first block start to its last wavefront end, read from
 * stamps the kernels write with the device's constant wall clock.  (The stop
 * events of hipExtLaunchKernelGGL land a few microseconds after a kernel's
 * end, which matters for kernels of tens of microseconds.)  Synchronizes the
 * stream of the last step.  SC_E_STATE if that step was not a timed one. */
SC_API sc_status slotcache_read_kernel_spans(sc_handle* h, double* us_out);

/* Counters of `layer`: the hit and miss counts that the pages read from the
 * engine's periodic cache statistics (page "GB300 GLM 5.3 Testing", section
 * "Sizing the context window: 256K, measured") and keep as hit/miss logs beside
 * every speed claim (same page, section "What changed in our policy").
 * Synchronizes the stream of the last step.  SC_E_DEVICE (with *out filled) when
 * a device-side check latched an error word on the layer. */
SC_API sc_status slotcache_stats(sc_handle* h, int32_t layer, sc_stats* out);

/* Slot map and LRU clock of `layer` (synchronizes): h_e2s int32[E] (slot or
 * -1), h_s2e int32[S] (expert or -1), h_key int64[S] (-1 = empty), h_step
 * (step counter).  Any output pointer may be NULL.  The slots are only a cache:
 * the backing store keeps the only full copy of every expert (page "TensorFold
 * GLM-5.3 explained"), so this state plus the backing store is a complete
 * checkpoint of the layer, and it is what the pages' "no stale slots" parity
 * check inspects (page "GB300 GLM 5.3 Testing", section "What changed in our
 * policy"). */
SC_API sc_status slotcache_read_state(sc_handle* h, int32_t layer, int32_t* h_e2s, int32_t* h_s2e,
                               int64_t* h_key, int64_t* h_step);

/* Restores a state read by slotcache_read_state (checkpoint / resume; the
 * backing store keeps the only full copy, page "TensorFold GLM-5.3 explained"):
 * copies the resident experts' blobs from the backing store into their slots
 * and writes maps, keys and step counter.  Counters and the event ring are left
 * as they are.  Synchronous.  SC_E_ARG, with nothing written, unless: the maps
 * are mutually inverse; empty slots have key -1; every occupied slot's key is a
 * clock value the layer could have stamped, -1 <= key < step * 16 * k (-1: never
 * referenced since it was filled); 0 <= step < 2^40; pinned slots keep their
 * experts. */
SC_API sc_status slotcache_write_state(sc_handle* h, int32_t layer, const int32_t* h_e2s,
                                const int32_t* h_s2e, const int64_t* h_key, int64_t step);

/* Miss events of `layer`, oldest first (synchronizes): the per-miss record
 * (step, expert in, slot, expert evicted) behind the pages' hit/miss logs (page
 * "GB300 GLM 5.3 Testing", section "What changed in our policy") and their
 * bit-exact churn comparisons (page "GLM 5.3 Testing: HBM Expert Allocation",
 * section "The build").  Copies up to `cap` records of the most recent
 * min(total, event_capacity) into h_buf; *n_out = records copied, *total =
 * events ever logged (total > event_capacity means the ring wrapped).  SC_E_ARG
 * if h_buf is NULL while records are available and cap > 0. */
SC_API sc_status slotcache_read_events(sc_handle* h, int32_t layer, sc_event* h_buf, size_t cap,
                                size_t* n_out, uint64_t* total);

/* Routing of the most recent step (synchronizes): h_ids int32[M*k],
 * h_w fp32[M*k] in (row, rank) order, *M_out = M, *bypass = 1 if the step
 * bypassed the cache.  Outputs may be NULL. */
SC_API sc_status slotcache_read_routing(sc_handle* h, int32_t* h_ids, float* h_w, int32_t* M_out,
                                 int32_t* bypass);

/* Message for the last non-OK status returned on this thread. */
SC_API const char* slotcache_last_error(void);

/* Frees the pinned backing store and the handle (synchronizes the device).
 * The caller's device buffers are not freed. */
SC_API void slotcache_destroy(sc_handle* h);

#ifdef __cplusplus
}
#endif

#endif /* SLOTCACHE_H */
