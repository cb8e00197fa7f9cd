// Host runtime of liblongflow.so: the C ABI declared in include/longflow.h.
//
// Static cache allocator (LongFlow Guide, §Static Memory Pre-Allocation and
// In-Place Eviction: one fixed buffer of B slots, never compacted): one
// hipMalloc at create time holds, for every (layer, sequence, KV head) pair,
//   K      [slots_pad][head_dim]  cache dtype (16-slot tiles, MFMA operand order)
//   V      [slots_pad][head_dim]  cache dtype
//   ||v||  [slots_pad]            float32 sidecar (l1, or l2)
//   fill                          int32 tokens held
//   victim                        int32 pending victim (deferred order)
//   split-K workspace  partial softmax states and arrival counters
//   per-sequence workspace  score vectors and arrival counters (one victim
//                           per sequence)
// and nothing is allocated afterwards. Validation happens on the host before
// anything is queued; fill levels are mirrored on the host (every decode step
// adds exactly one token per pair) so no call has to read the device, and the
// split count of each launch is planned from them.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <numeric>
#include <vector>

#include "../../include/longflow.h"
#include "../../include/longflow_probe.h"
#include "lf_internal.h"

struct lf_cache {
  lf_config cfg;
  lf::Geometry geo;
  int device;
  size_t bytes;
  void* base;
  char* k;
  char* v;
  float* vnorm;
  int32_t* fill;
  int32_t* victim;
  int32_t* order;        // [num_layers][batch]: FULL mode launch order of the sequences
  int64_t layer_pairs;   // batch * num_kv_heads
  size_t elem_bytes;
  std::vector<int32_t> fill_host;  // [num_layers][batch]
  lf::SplitWork work;              // split-K workspace (shared by the layers)
  int32_t max_splits;              // 1: no split launches
  int32_t forced_splits;           // 0: plan automatically
  int32_t forced_waves;            // 0: plan automatically
  int32_t forced_loop;             // 0: plan automatically, 1: phased, 2: interleaved
  int32_t forced_grid;             // 0: plan automatically, -1: one workgroup per pair, > 0: cap
  int32_t forced_stream;           // 0: plan automatically, > 0: stream launch of that many tiles
  int32_t sk_rows;                 // workspace rows for the cut pairs of a stream launch
  int32_t sk_stride;               // partials per workspace row
  int32_t cus;                     // compute units of the device
  size_t lds_limit;                // LDS bytes one workgroup may use
  size_t lds_per_cu;               // LDS bytes of one compute unit
};

namespace {

constexpr size_t kAlign = 256;
constexpr int kSlotAlign = 64;

struct Layout {
  size_t k_off, v_off, vn_off, fill_off, victim_off, order_off, part_off, logit_off, arrive_off,
      score_off, seq_arrive_off, new_norm_off, total;
  int32_t slots_pad;
  int64_t pair_elems;
};

bool mul_ok(size_t a, size_t b, size_t* r) { return !__builtin_mul_overflow(a, b, r); }
bool add_ok(size_t a, size_t b, size_t* r) { return !__builtin_add_overflow(a, b, r); }
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

lf_status validate(const lf_config* c) {
  if (!c) return LF_ERR_INVALID_ARG;
  if (c->num_layers < 1 || c->batch < 1 || c->num_q_heads < 1 || c->num_kv_heads < 1 ||
      c->head_dim < 1 || c->budget < 1)
    return LF_ERR_INVALID_ARG;
  if (c->num_q_heads % c->num_kv_heads) return LF_ERR_INVALID_ARG;
  if (c->sink_size < 0 || c->sink_size >= c->budget) return LF_ERR_INVALID_ARG;
  if (!(c->softmax_scale >= 0.0f) || !std::isfinite(c->softmax_scale)) return LF_ERR_INVALID_ARG;
  if (c->dtype != LF_DTYPE_F32 && c->dtype != LF_DTYPE_BF16) return LF_ERR_INVALID_ARG;
  if (c->mode != LF_MODE_EVICT && c->mode != LF_MODE_FULL) return LF_ERR_INVALID_ARG;
  if (c->order != LF_ORDER_SAME_STEP && c->order != LF_ORDER_DEFERRED) return LF_ERR_INVALID_ARG;
  if (c->scope != LF_SCOPE_KV_HEAD && c->scope != LF_SCOPE_SEQUENCE) return LF_ERR_INVALID_ARG;
  if (c->norm != LF_NORM_L1 && c->norm != LF_NORM_L2) return LF_ERR_INVALID_ARG;
  if (c->mode == LF_MODE_FULL && (c->order || c->scope || c->norm)) return LF_ERR_INVALID_ARG;
  if (c->head_dim != 64 && c->head_dim != 128) return LF_ERR_UNSUPPORTED;
  const int g = c->num_q_heads / c->num_kv_heads;
  if (g != 1 && g != 2 && g != 4) return LF_ERR_UNSUPPORTED;
  if (c->budget > (1 << 30) - kSlotAlign) return LF_ERR_UNSUPPORTED;
  {
    // The kernels address one pair's K and V rows with 32-bit byte offsets.
    const int64_t slots_pad = (static_cast<int64_t>(c->budget) + kSlotAlign - 1) / kSlotAlign * kSlotAlign;
    const int64_t row_bytes = static_cast<int64_t>(c->head_dim) * (c->dtype == LF_DTYPE_F32 ? 4 : 2);
    if (slots_pad * row_bytes > int64_t{0xffffffff}) return LF_ERR_UNSUPPORTED;
  }
  if (c->scope == LF_SCOPE_SEQUENCE) {
    // The deciding workgroup addresses a sequence's score vectors with 32-bit
    // offsets.
    const int64_t slots_pad = (static_cast<int64_t>(c->budget) + kSlotAlign - 1) / kSlotAlign * kSlotAlign;
    if (static_cast<int64_t>(c->num_kv_heads) * slots_pad * 4 >= (int64_t{1} << 31))
      return LF_ERR_UNSUPPORTED;
  }
  return LF_OK;
}

lf::Geometry geometry(const lf_config* c) {
  lf::Geometry g;
  g.batch = c->batch;
  g.num_q_heads = c->num_q_heads;
  g.num_kv_heads = c->num_kv_heads;
  g.group = c->num_q_heads / c->num_kv_heads;
  g.head_dim = c->head_dim;
  g.budget = c->budget;
  g.sink_size = c->sink_size;
  g.slots_pad = (c->budget + kSlotAlign - 1) / kSlotAlign * kSlotAlign;
  g.dtype = c->dtype;
  g.mode = c->mode;
  g.order = c->order;
  g.scope = c->scope;
  g.norm = c->norm;
  g.pair_elems = static_cast<int64_t>(g.slots_pad) * c->head_dim;
  g.scale = c->softmax_scale > 0.0f ? c->softmax_scale
                                    : static_cast<float>(1.0 / std::sqrt(static_cast<double>(c->head_dim)));
  return g;
}

// Workspace rows for the cut pairs of stream launches on the evicting main
// path (same-step order, one victim per KV head): the most pairs the stream
// rule of plan_stream cuts on a device of kStreamCusRef compute units, at
// most kStreamRows.
// Layers with a split-K workspace (max_splits > 1) use that one instead.
int32_t stream_rows(const lf_config* c, int32_t max_splits) {
  const int64_t pairs = static_cast<int64_t>(c->batch) * c->num_kv_heads;
  if (max_splits > 1 || c->mode != LF_MODE_EVICT || c->order != LF_ORDER_SAME_STEP ||
      c->scope != LF_SCOPE_KV_HEAD || pairs <= lf::kStreamCusRef)
    return 0;
  // just past one round of 8-wave workgroups (room = CUs), or past whole
  // rounds of 4-wave ones (room = 2 CUs)
  int64_t rows = 0;
  const int64_t cus = lf::kStreamCusRef;
  if (pairs > cus && (pairs - cus) * 4 <= cus) rows = pairs - cus;
  const int64_t cut = pairs % (2 * cus);
  if (pairs > 2 * cus && cut * 4 <= 2 * cus) rows = std::max(rows, cut);
  return static_cast<int32_t>(std::min<int64_t>(rows, lf::kStreamRows));
}

lf_status layout(const lf_config* c, int32_t max_splits, Layout* L) {
  const lf::Geometry g = geometry(c);
  const size_t elem = c->dtype == LF_DTYPE_F32 ? 4 : 2;
  size_t pairs, kv, vn, fl, t;
  if (!mul_ok(static_cast<size_t>(c->num_layers), static_cast<size_t>(c->batch), &pairs) ||
      !mul_ok(pairs, static_cast<size_t>(c->num_kv_heads), &pairs))
    return LF_ERR_UNSUPPORTED;
  if (!mul_ok(pairs, static_cast<size_t>(g.pair_elems), &kv) || !mul_ok(kv, elem, &kv))
    return LF_ERR_UNSUPPORTED;
  if (!mul_ok(pairs, static_cast<size_t>(g.slots_pad), &vn) || !mul_ok(vn, 4, &vn))
    return LF_ERR_UNSUPPORTED;
  if (!mul_ok(pairs, 4, &fl)) return LF_ERR_UNSUPPORTED;
  L->slots_pad = g.slots_pad;
  L->pair_elems = g.pair_elems;
  L->k_off = 0;
  if (!add_ok(align_up(kv), 0, &t)) return LF_ERR_UNSUPPORTED;
  L->v_off = t;
  if (!add_ok(L->v_off, align_up(kv), &t)) return LF_ERR_UNSUPPORTED;
  L->vn_off = t;
  if (!add_ok(L->vn_off, align_up(vn), &t)) return LF_ERR_UNSUPPORTED;
  L->fill_off = t;
  if (!add_ok(L->fill_off, align_up(fl), &t)) return LF_ERR_UNSUPPORTED;
  L->victim_off = t;
  if (!add_ok(L->victim_off, align_up(fl), &t)) return LF_ERR_UNSUPPORTED;
  // FULL mode: each layer's launch order of its sequences.
  L->order_off = t;
  if (!add_ok(L->order_off, align_up(c->mode == LF_MODE_FULL
                                          ? static_cast<size_t>(c->num_layers) * c->batch * 4 : 0), &t))
    return LF_ERR_UNSUPPORTED;
  // Split-K workspace for one layer (the layers run one after another):
  // split launches (rows = pairs, max_splits partials each), or the cut
  // pairs of stream launches (stream_rows rows of kMaxSplits partials).
  size_t layer_pairs = static_cast<size_t>(c->batch) * c->num_kv_heads;
  const size_t srows = static_cast<size_t>(stream_rows(c, max_splits));
  size_t ws = max_splits > 1 ? layer_pairs * max_splits : srows * lf::kMaxSplits;
  const size_t logit_rows = max_splits > 1 ? layer_pairs : srows;
  const size_t logits = (max_splits > 1 || srows > 0) && c->mode == LF_MODE_EVICT
      ? logit_rows * static_cast<size_t>(g.slots_pad) * g.group * 4 : 0;
  L->part_off = t;
  if (!add_ok(L->part_off, align_up(ws * lf::split_part_floats(g) * 4), &t)) return LF_ERR_UNSUPPORTED;
  L->logit_off = t;
  if (!add_ok(L->logit_off, align_up(logits), &t)) return LF_ERR_UNSUPPORTED;
  L->arrive_off = t;
  if (!add_ok(L->arrive_off, align_up(max_splits > 1 ? layer_pairs * 4 : srows * 4), &t))
    return LF_ERR_UNSUPPORTED;
  // One victim per sequence: each pair's score vector for one layer launch.
  const bool shared = c->scope == LF_SCOPE_SEQUENCE;
  L->score_off = t;
  if (!add_ok(L->score_off, align_up(shared ? layer_pairs * static_cast<size_t>(g.slots_pad) * 4 : 0), &t))
    return LF_ERR_UNSUPPORTED;
  L->seq_arrive_off = t;
  if (!add_ok(L->seq_arrive_off, align_up(shared ? static_cast<size_t>(c->batch) * 4 : 0), &t))
    return LF_ERR_UNSUPPORTED;
  L->new_norm_off = t;
  if (!add_ok(L->new_norm_off, align_up(shared ? layer_pairs * 4 : 0), &t)) return LF_ERR_UNSUPPORTED;
  L->total = t;
  return LF_OK;
}

// Largest split count a cache can use (sizes its workspace): none once the
// layer has kSplitPairsBelow pairs, else kSplitGridTarget / pairs, capped at
// kMaxSplits. Decided from the configuration alone, so that lf_cache_bytes
// needs no device.
int32_t max_splits_for(const lf_config* c) {
  const int64_t pairs = static_cast<int64_t>(c->batch) * c->num_kv_heads;
  if (pairs <= 0 || pairs >= lf::kSplitPairsBelow) return 1;
  const int64_t s = lf::kSplitGridTarget / pairs;
  return static_cast<int32_t>(std::max<int64_t>(1, std::min<int64_t>(s, lf::kMaxSplits)));
}

lf::LayerPtrs layer_ptrs(const lf_cache* c, int32_t layer) {
  lf::LayerPtrs p;
  const int64_t pair0 = static_cast<int64_t>(layer) * c->layer_pairs;
  p.k = c->k + pair0 * c->geo.pair_elems * static_cast<int64_t>(c->elem_bytes);
  p.v = c->v + pair0 * c->geo.pair_elems * static_cast<int64_t>(c->elem_bytes);
  p.vnorm = c->vnorm + pair0 * c->geo.slots_pad;
  p.fill = c->fill + pair0;
  p.victim = c->victim + pair0;
  p.order = c->order ? c->order + static_cast<int64_t>(layer) * c->cfg.batch : nullptr;
  return p;
}

// FULL mode: one layer's sequences in launch order, longest first (ties by
// index), written to the device. Workgroups are dispatched in index order, so
// the longest pairs start first and the short ones fill the last round.
// Decode steps add one token to every sequence, which keeps the order; only
// prefill and recycling change it.
hipError_t write_order(const lf_cache* c, int32_t layer, hipStream_t st) {
  if (!c->order) return hipSuccess;
  const int32_t batch = c->cfg.batch;
  const int32_t* fh = c->fill_host.data() + static_cast<size_t>(layer) * batch;
  std::vector<int32_t> seq(batch);
  std::iota(seq.begin(), seq.end(), 0);
  std::stable_sort(seq.begin(), seq.end(), [fh](int32_t a, int32_t b) { return fh[a] > fh[b]; });
  int32_t* dst = c->order + static_cast<int64_t>(layer) * batch;
  for (int32_t first = 0; first < batch; first += lf::kOrderPerLaunch) {
    const int32_t n = std::min<int32_t>(lf::kOrderPerLaunch, batch - first);
    const hipError_t e = lf::launch_set_order(dst, seq.data() + first, first, n, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Makes the cache's device current for the length of one call and gives the
// caller's current device back afterwards.
class DeviceScope {
 public:
  explicit DeviceScope(int device) {
    if (hipGetDevice(&prev_) != hipSuccess) {
      ok_ = false;
      return;
    }
    if (prev_ != device) ok_ = switched_ = hipSetDevice(device) == hipSuccess;
  }
  ~DeviceScope() {
    if (switched_) (void)hipSetDevice(prev_);
  }
  DeviceScope(const DeviceScope&) = delete;
  DeviceScope& operator=(const DeviceScope&) = delete;
  bool ok() const { return ok_; }

 private:
  int prev_ = -1;
  bool ok_ = true;
  bool switched_ = false;
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Launch shape of one decode step: workgroups per pair (split-K) and waves
// per workgroup.
//   - A layer with at least as many pairs as compute units runs one
//     workgroup per pair.
//   - With fewer pairs, each pair splits over up to cus / pairs workgroups
//     (at most max_splits, at least kMinSplitSlots slots per split of the
//     fullest pair), so the launch holds about one workgroup per CU.
//   - Workgroups that stream at most kInterleaveSlots slots run the
//     interleaved loop (K and V of each tile together); longer streams run
//     the phased loop (K, then V).
//   - A launch of at most one workgroup per CU uses 8 waves per workgroup,
//     otherwise 4 (two workgroups per CU). This needs the 8-wave
//     workgroup's LDS to fit, and at least 8 tiles per workgroup.
//   - A one-workgroup-per-pair launch of the evicting main path (4 waves,
//     no variant) may run as a stream launch instead (plan_stream).
// A forced split count (lf_cache_set_splits) wins within max_splits.
struct LaunchShape {
  int32_t splits;
  int32_t waves;
  bool ilv;  // interleaved loop (short streams) instead of the phased one
};

LaunchShape plan_launch(const lf_cache* c, int32_t n_max) {
  const int64_t pairs = c->layer_pairs;
  int32_t s = 1;
  if (c->max_splits > 1) {
    if (c->forced_splits > 0) {
      s = std::min(c->forced_splits, c->max_splits);
    } else if (pairs < c->cus) {
      const int64_t by_grid = std::max<int64_t>(1, c->cus / pairs);
      const int32_t by_work = std::max(1, n_max / lf::kMinSplitSlots);
      s = static_cast<int32_t>(std::min<int64_t>({c->max_splits, by_grid, by_work}));
    }
  }
  // Slots one workgroup streams: short streams take the interleaved loop.
  const int32_t per_wg = (n_max + s - 1) / s;
  bool ilv = per_wg <= lf::kInterleaveSlots;
  if (c->forced_loop > 0) ilv = c->forced_loop == 2;
  const size_t dyn = s > 1 ? lf::decode_split_lds_bytes(c->geo, s, ilv) : lf::decode_lds_bytes(c->geo, ilv);
  const bool fits8 = dyn + lf::decode_static_lds_bytes(c->geo, 8) <= c->lds_limit;
  // 8 waves only when every wave has a 16-slot tile to stream (a 64-slot
  // pair on 8 waves leaves half of them idle: 5.2 against 4.8 us per step).
  int32_t waves = pairs * s <= c->cus && (per_wg + 15) / 16 >= 8 ? 8 : 4;
  if (c->forced_waves > 0) waves = c->forced_waves;
  if (waves == 8 && !fits8) waves = 4;
  return {s, waves, ilv};
}

// Resident 4-wave decode workgroups per compute unit: two (the kernels'
// launch bounds) when their LDS fits the compute unit twice, else one.
int32_t resident_4wave(const lf_cache* c, bool ilv) {
  const size_t per_wg = lf::decode_lds_bytes(c->geo, ilv) + lf::decode_static_lds_bytes(c->geo, 4);
  return 2 * per_wg <= c->lds_per_cu ? 2 : 1;
}

// Stream launch of the evicting main path (no split, no variant), or grid = 0
// for one workgroup per pair. With R workgroups resident at once, P pairs
// take ceil(P / R) rounds of whole pairs, and a part-full last round leaves
// the device partly idle.
//   - Just past k whole rounds (k R < P <= (k + 0.25) R): every workgroup
//     takes its k whole pairs of those rounds in turn, then an equal run
//     (at least kStreamMinTiles tiles) of the remaining pairs' tiles; pairs
//     cut between workgroups combine their parts as split-K does. Just past
//     one round of 8-wave workgroups (one per compute unit: cus < P <= 1.25
//     cus) the launch switches to 8 waves for this; past k rounds of 4-wave
//     workgroups (two per compute unit) it keeps 4. Needs workspace rows for
//     the cut pairs. Measured on the Llama-8B layer, the gain falls from
//     10-19% with a few cut pairs to nothing at 0.3 R.
//   - Two rounds of 4-wave workgroups with the second 40-85% full:
//     ceil(P / 2) workgroups taking two whole pairs each.
//   - Otherwise one workgroup per pair.
// No pair is cut into more than `stride` parts. Overrides: forced_stream > 0
// streams every pair with that many tiles per workgroup (no whole pairs
// first); forced_grid > 0 takes whole pairs in turn on that many
// workgroups; forced_grid < 0 keeps one workgroup per pair.
// What plan_stream decides from, apart from the cache: the device, the
// layer's workspace and the overrides (also the input of
// lf_probe_stream_plan).
struct StreamInputs {
  int64_t pairs;
  int32_t n_max;
  int32_t cus;
  int32_t resident4;   // resident 4-wave workgroups per CU
  bool fits8;          // an 8-wave workgroup's LDS fits
  int32_t rows;        // workspace rows for cut pairs
  int32_t stride;      // partials per row
  int32_t forced_stream, forced_grid, forced_waves;
};

lf::GridPlan stream_plan(const StreamInputs& in, bool* eight_waves) {
  lf::GridPlan g;
  *eight_waves = false;
  if (in.forced_grid < 0) return g;
  const int64_t pairs = in.pairs;
  const int64_t tn = std::max<int64_t>(1, (static_cast<int64_t>(in.n_max) + 15) / 16);
  const int64_t stride = in.stride;
  // tiles per share so that no pair is cut into more than `stride` parts
  const int64_t q_min = stride > 1 ? (tn + stride - 2) / (stride - 1) : tn;
  auto stream = [&](int64_t first, int64_t q, int64_t grid_min) {
    const int64_t run = (pairs - first) * tn;
    q = std::max(q, q_min);
    g.sk_first = static_cast<int>(first);
    g.sk_pairs = static_cast<int>(pairs - first);
    g.sk_tiles = static_cast<int>(tn);
    g.sk_q = static_cast<int>(q);
    g.sk_wgs = static_cast<int>((run + q - 1) / q);
    g.sk_stride = static_cast<int>(stride);
    g.grid = static_cast<int>(std::max<int64_t>(grid_min, g.sk_wgs));
  };
  if (in.forced_stream > 0) {
    if (pairs <= in.rows && stride > 1) stream(0, in.forced_stream, 1);
    return g;
  }
  if (in.forced_grid > 0) {
    if (in.forced_grid < pairs) {
      g.grid = in.forced_grid;
      g.sk_first = static_cast<int>(pairs);
    }
    return g;
  }
  // k whole rounds of `room` workgroups (each workgroup takes k whole pairs
  // in turn), the remaining pairs cut into runs
  auto past_whole_rounds = [&](int64_t room, int64_t max_rounds) {
    const int64_t k = pairs / room;
    const int64_t cut = pairs - k * room;
    if (k < 1 || k > max_rounds || cut <= 0 || cut > in.rows || stride <= 1 || cut * 4 > room)
      return false;
    const int64_t run = cut * tn;
    const int64_t wgs = std::max<int64_t>(1, std::min<int64_t>(room, run / lf::kStreamMinTiles));
    stream(k * room, std::max<int64_t>((run + wgs - 1) / wgs, lf::kStreamMinTiles), room);
    return true;
  };
  if (in.forced_waves == 0 && in.fits8 && past_whole_rounds(in.cus, 1)) {
    *eight_waves = true;
    return g;
  }
  const int64_t room = static_cast<int64_t>(in.resident4) * in.cus;
  if (room <= in.cus || pairs <= in.cus) return g;
  if (past_whole_rounds(room, pairs)) return g;
  const int64_t last = pairs - room;  // pairs of a second round
  if (last > 0 && last <= room && last * 10 >= room * 4 && last * 20 <= room * 17) {
    g.grid = static_cast<int>((pairs + 1) / 2);
    g.sk_first = static_cast<int>(pairs);
  }
  return g;
}

lf::GridPlan plan_stream(const lf_cache* c, LaunchShape* shape, int32_t n_max) {
  const lf::Geometry& geo = c->geo;
  // one-workgroup-per-pair launches of 4 waves on the evicting main path
  // (a forced stream launch also takes an 8-wave shape)
  if (shape->splits != 1 || geo.mode != LF_MODE_EVICT || geo.order != 0 || geo.scope != 0 ||
      (shape->waves != 4 && c->forced_stream == 0))
    return lf::GridPlan{};
  StreamInputs in;
  in.pairs = c->layer_pairs;
  in.n_max = n_max;
  in.cus = c->cus;
  in.resident4 = resident_4wave(c, shape->ilv);
  in.fits8 = lf::decode_lds_bytes(geo, shape->ilv) + lf::decode_static_lds_bytes(geo, 8) <= c->lds_limit;
  in.rows = c->sk_rows;
  in.stride = c->sk_stride;
  in.forced_stream = c->forced_stream;
  in.forced_grid = c->forced_grid;
  in.forced_waves = c->forced_waves;
  bool eight = false;
  const lf::GridPlan g = stream_plan(in, &eight);
  if (eight) shape->waves = 8;
  return g;
}

// Workspace of one decode launch carved out of the device's static scratch:
// counters at fixed words of the counter area, the rest after it. Returns
// false if the launch needs more than the array holds.
bool scratch_work(const lf_cache* c, char* base, int32_t splits, const lf::GridPlan& plan,
                  lf::SplitWork* w) {
  const lf::Geometry& g = c->geo;
  const bool split = splits > 1;
  const bool cut = plan.grid > 0 && plan.sk_pairs > 0;  // stream launch with cut pairs
  // workspace rows: every pair (split-K) or the stream launch's cut pairs
  const size_t pairs = static_cast<size_t>(c->layer_pairs);
  const size_t rows = split ? pairs : cut ? static_cast<size_t>(plan.sk_pairs) : 0;
  const size_t per_row = split ? static_cast<size_t>(splits) : static_cast<size_t>(plan.sk_stride);
  const bool shared = g.scope == LF_SCOPE_SEQUENCE;
  if (rows > static_cast<size_t>(lf::kScratchSeqCounterWord)) return false;
  if (shared && (static_cast<size_t>(lf::kScratchSeqCounterWord) + g.batch) * 4 > lf::kScratchCounterBytes)
    return false;
  size_t off = lf::kScratchCounterBytes;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes);
    return base + at;
  };
  // Each size is at most the cache's own K region, so none overflows.
  const size_t part = rows * per_row * lf::split_part_floats(g) * 4;
  const size_t logit = g.mode == LF_MODE_EVICT ? rows * g.slots_pad * g.group * 4 : 0;
  const size_t score = shared ? pairs * g.slots_pad * 4 : 0;
  const size_t nnorm = shared ? pairs * 4 : 0;
  if (part > lf::kScratchBytes || logit > lf::kScratchBytes || score > lf::kScratchBytes) return false;
  w->part = reinterpret_cast<float*>(take(part));
  w->logit = reinterpret_cast<float*>(take(logit));
  w->score = reinterpret_cast<float*>(take(score));
  w->new_norm = reinterpret_cast<float*>(take(nnorm));
  w->arrive = reinterpret_cast<int32_t*>(base);
  w->seq_arrive = reinterpret_cast<int32_t*>(base) + lf::kScratchSeqCounterWord;
  return off <= lf::kScratchBytes;
}

// Optional per-workgroup timing of one decode launch (measurement probe).
struct Timing {
  uint64_t* records;   // device [capacity][4]
  int64_t capacity;
  int32_t* workgroups; // host: the launch's workgroup count
  uint64_t* phases;    // device [capacity][8], or null
};

// One decode step of one layer; `static_scratch` takes the launch's
// workspace from the device's static array instead of the cache's own;
// `timing` (may be null) asks for per-workgroup timing records.
lf_status decode_step(lf_cache* c, int32_t layer, const void* q, const void* k_new, const void* v_new,
                      void* out, int32_t* evicted_slot, void* stream, bool static_scratch,
                      const Timing* timing = nullptr) {
  if (!c || !q || !k_new || !v_new || !out || !evicted_slot || layer < 0 ||
      layer >= c->cfg.num_layers)
    return LF_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out))
    return LF_ERR_INVALID_ARG;
  int32_t* fh = c->fill_host.data() + static_cast<size_t>(layer) * c->cfg.batch;
  if (c->cfg.mode == LF_MODE_FULL) {
    for (int32_t b = 0; b < c->cfg.batch; ++b)
      if (fh[b] >= c->cfg.budget) return LF_ERR_CAPACITY;
  }
  int32_t n_max = 0;
  for (int32_t b = 0; b < c->cfg.batch; ++b) n_max = std::max(n_max, fh[b]);
  LaunchShape shape = plan_launch(c, n_max);
  const lf::GridPlan grid = plan_stream(c, &shape, n_max);
  lf::SplitWork work = c->work;
  const int64_t wgs = grid.grid > 0 ? grid.grid : c->layer_pairs * shape.splits;
  if (timing) {
    if (!timing->records || !timing->workgroups || timing->capacity < wgs) return LF_ERR_INVALID_ARG;
    work.wg_clock = timing->records;
    work.wg_phase = timing->phases;
  }
  if (static_scratch) {
    char* base = static_cast<char*>(lf::scratch_ptr(c->device));
    if (!base) return LF_ERR_HIP;  // set up by lf_cache_create on this device
    if (!scratch_work(c, base, shape.splits, grid, &work)) return LF_ERR_SCRATCH;
  }
  DeviceScope dev(c->device);
  if (!dev.ok()) return LF_ERR_HIP;
  const lf::LayerPtrs p = layer_ptrs(c, layer);
  if (lf::launch_decode(c->geo, p, work, shape.splits, shape.waves, shape.ilv, grid, q, k_new, v_new,
                        out, evicted_slot, static_cast<hipStream_t>(stream)) != hipSuccess) {
    (void)hipGetLastError();
    return LF_ERR_HIP;
  }
  if (timing) *timing->workgroups = static_cast<int32_t>(wgs);
  for (int32_t b = 0; b < c->cfg.batch; ++b)
    if (fh[b] < c->cfg.budget) ++fh[b];
  return LF_OK;
}

}  // namespace

extern "C" {

const char* lf_status_str(lf_status s) {
  switch (s) {
    case LF_OK: return "LF_OK";
    case LF_ERR_INVALID_ARG: return "LF_ERR_INVALID_ARG";
    case LF_ERR_UNSUPPORTED: return "LF_ERR_UNSUPPORTED";
    case LF_ERR_CAPACITY: return "LF_ERR_CAPACITY";
    case LF_ERR_OOM: return "LF_ERR_OOM";
    case LF_ERR_HIP: return "LF_ERR_HIP";
    case LF_ERR_SCRATCH: return "LF_ERR_SCRATCH";
  }
  return "LF_ERR_UNKNOWN";
}

lf_status lf_cache_bytes(const lf_config* cfg, size_t* bytes) {
  if (!bytes) return LF_ERR_INVALID_ARG;
  lf_status s = validate(cfg);
  if (s != LF_OK) return s;
  Layout L;
  // The split workspace is sized for the most splits that could be planned
  // (an upper bound that needs no device query).
  s = layout(cfg, max_splits_for(cfg), &L);
  if (s != LF_OK) return s;
  *bytes = L.total;
  return LF_OK;
}

lf_status lf_cache_create(const lf_config* cfg, lf_cache** out) {
  if (!out) return LF_ERR_INVALID_ARG;
  *out = nullptr;
  lf_status s = validate(cfg);
  if (s != LF_OK) return s;
  const lf::Geometry geo = geometry(cfg);
  // The phased loop needs the most LDS (it also keeps the scores of one
  // victim per sequence); every launch then fits either loop.
  const size_t lds = lf::decode_lds_bytes(geo, false);
  if (lds == 0) return LF_ERR_UNSUPPORTED;
  int device = -1;
  if (hipGetDevice(&device) != hipSuccess) {
    (void)hipGetLastError();
    return LF_ERR_HIP;
  }
  if (lds > lf::device_lds_limit()) return LF_ERR_UNSUPPORTED;
  const int32_t max_splits = max_splits_for(cfg);
  Layout L;
  s = layout(cfg, max_splits, &L);
  if (s != LF_OK) return s;

  lf_cache* c = new (std::nothrow) lf_cache();
  if (!c) return LF_ERR_OOM;
  try {
    c->fill_host.assign(static_cast<size_t>(cfg->num_layers) * cfg->batch, 0);
  } catch (...) {
    delete c;
    return LF_ERR_OOM;
  }
  c->cfg = *cfg;
  c->geo = geo;
  c->bytes = L.total;
  c->elem_bytes = cfg->dtype == LF_DTYPE_F32 ? 4 : 2;
  c->layer_pairs = static_cast<int64_t>(cfg->batch) * cfg->num_kv_heads;
  c->device = device;
  void* base = nullptr;
  hipError_t e = hipMalloc(&base, L.total);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    delete c;
    return e == hipErrorOutOfMemory ? LF_ERR_OOM : LF_ERR_HIP;
  }
  e = hipMemsetAsync(base, 0, L.total, nullptr);
  if (e == hipSuccess && cfg->mode == LF_MODE_FULL) {
    // every sequence starts empty: the launch order is the identity
    c->order = reinterpret_cast<int32_t*>(static_cast<char*>(base) + L.order_off);
    for (int32_t l = 0; l < cfg->num_layers && e == hipSuccess; ++l)
      e = write_order(c, l, nullptr);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(nullptr);
  // The device's static scratch (lf_decode_step_noalloc) is set up here,
  // outside any stream capture, once per device.
  if (e == hipSuccess) e = lf::scratch_setup(device);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    (void)hipFree(base);
    delete c;
    return LF_ERR_HIP;
  }
  c->base = base;
  c->k = static_cast<char*>(base) + L.k_off;
  c->v = static_cast<char*>(base) + L.v_off;
  c->vnorm = reinterpret_cast<float*>(static_cast<char*>(base) + L.vn_off);
  c->fill = reinterpret_cast<int32_t*>(static_cast<char*>(base) + L.fill_off);
  c->victim = reinterpret_cast<int32_t*>(static_cast<char*>(base) + L.victim_off);
  c->order = cfg->mode == LF_MODE_FULL
                 ? reinterpret_cast<int32_t*>(static_cast<char*>(base) + L.order_off)
                 : nullptr;
  c->work.part = reinterpret_cast<float*>(static_cast<char*>(base) + L.part_off);
  c->work.logit = reinterpret_cast<float*>(static_cast<char*>(base) + L.logit_off);
  c->work.arrive = reinterpret_cast<int32_t*>(static_cast<char*>(base) + L.arrive_off);
  c->work.score = reinterpret_cast<float*>(static_cast<char*>(base) + L.score_off);
  c->work.seq_arrive = reinterpret_cast<int32_t*>(static_cast<char*>(base) + L.seq_arrive_off);
  c->work.new_norm = reinterpret_cast<float*>(static_cast<char*>(base) + L.new_norm_off);
  c->max_splits = max_splits;
  c->forced_splits = 0;
  c->forced_waves = 0;
  c->forced_loop = 0;
  c->forced_grid = 0;
  c->forced_stream = 0;
  c->sk_rows = max_splits > 1 ? static_cast<int32_t>(c->layer_pairs) : stream_rows(cfg, max_splits);
  c->sk_stride = max_splits > 1 ? max_splits : lf::kMaxSplits;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus < 1)
    cus = 256;
  c->cus = cus;
  c->lds_limit = lf::device_lds_limit();
  int lds_cu = 0;
  if (hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, device) !=
          hipSuccess ||
      lds_cu < 1) {
    (void)hipGetLastError();
    lds_cu = 160 * 1024;
  }
  c->lds_per_cu = static_cast<size_t>(lds_cu);
  *out = c;
  return LF_OK;
}

void lf_cache_destroy(lf_cache* c) {
  if (!c) return;
  if (c->base) {
    DeviceScope dev(c->device);
    (void)hipFree(c->base);
  }
  delete c;
}

lf_status lf_cache_view(const lf_cache* c, int32_t layer, lf_view* view) {
  if (!c || !view || layer < 0 || layer >= c->cfg.num_layers) return LF_ERR_INVALID_ARG;
  const lf::LayerPtrs p = layer_ptrs(c, layer);
  view->k = p.k;
  view->v = p.v;
  view->vnorm = p.vnorm;
  view->fill = p.fill;
  view->victim = p.victim;
  view->pair_stride = c->geo.pair_elems;
  view->slots_padded = c->geo.slots_pad;
  view->elem_bytes = static_cast<int32_t>(c->elem_bytes);
  return LF_OK;
}

lf_status lf_cache_snapshot(const lf_cache* c, int32_t layer, void* k, void* v, float* vnorm,
                            int32_t* fill, int32_t* victim, void* stream) {
  if (!c || layer < 0 || layer >= c->cfg.num_layers) return LF_ERR_INVALID_ARG;
  DeviceScope dev(c->device);
  if (!dev.ok()) return LF_ERR_HIP;
  const lf::LayerPtrs p = layer_ptrs(c, layer);
  const size_t kv_bytes = static_cast<size_t>(c->layer_pairs) * c->geo.pair_elems * c->elem_bytes;
  const size_t vn_bytes = static_cast<size_t>(c->layer_pairs) * c->geo.slots_pad * sizeof(float);
  const size_t fill_bytes = static_cast<size_t>(c->layer_pairs) * sizeof(int32_t);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const struct { void* dst; const void* src; size_t n; } copies[] = {
      {k, p.k, kv_bytes}, {v, p.v, kv_bytes}, {vnorm, p.vnorm, vn_bytes}, {fill, p.fill, fill_bytes},
      {victim, p.victim, fill_bytes}};
  for (const auto& cp : copies) {
    if (!cp.dst) continue;
    if (hipMemcpyAsync(cp.dst, cp.src, cp.n, hipMemcpyDeviceToDevice, st) != hipSuccess)
      return LF_ERR_HIP;
  }
  return LF_OK;
}

lf_status lf_cache_set_splits(lf_cache* c, int32_t splits) {
  if (!c || splits < 0) return LF_ERR_INVALID_ARG;
  c->forced_splits = splits;
  return LF_OK;
}

lf_status lf_cache_set_waves(lf_cache* c, int32_t waves) {
  if (!c || (waves != 0 && waves != 4 && waves != 8)) return LF_ERR_INVALID_ARG;
  c->forced_waves = waves;
  return LF_OK;
}

lf_status lf_cache_set_loop(lf_cache* c, int32_t loop) {
  if (!c || loop < 0 || loop > 2) return LF_ERR_INVALID_ARG;
  c->forced_loop = loop;
  return LF_OK;
}

lf_status lf_cache_set_grid(lf_cache* c, int32_t workgroups) {
  if (!c || workgroups < -1) return LF_ERR_INVALID_ARG;
  c->forced_grid = workgroups;
  return LF_OK;
}

lf_status lf_cache_set_stream(lf_cache* c, int32_t tiles) {
  if (!c || tiles < 0) return LF_ERR_INVALID_ARG;
  c->forced_stream = tiles;
  return LF_OK;
}

lf_status lf_cache_max_splits(const lf_cache* c, int32_t* max_splits) {
  if (!c || !max_splits) return LF_ERR_INVALID_ARG;
  *max_splits = c->max_splits;
  return LF_OK;
}

lf_status lf_fill_levels(const lf_cache* c, int32_t layer, int32_t* fill_host) {
  if (!c || !fill_host || layer < 0 || layer >= c->cfg.num_layers) return LF_ERR_INVALID_ARG;
  std::memcpy(fill_host, c->fill_host.data() + static_cast<size_t>(layer) * c->cfg.batch,
              sizeof(int32_t) * c->cfg.batch);
  return LF_OK;
}

lf_status lf_prefill_fill(lf_cache* c, int32_t layer, const void* k, const void* v,
                          const int32_t* n_per_seq, int32_t n_max, void* stream) {
  if (!c || !n_per_seq || layer < 0 || layer >= c->cfg.num_layers || n_max < 0)
    return LF_ERR_INVALID_ARG;
  if (n_max > 0 && (!k || !v || !aligned16(k) || !aligned16(v))) return LF_ERR_INVALID_ARG;
  for (int32_t b = 0; b < c->cfg.batch; ++b) {
    if (n_per_seq[b] < -1 || n_per_seq[b] > n_max) return LF_ERR_INVALID_ARG;
    if (n_per_seq[b] > c->cfg.budget) return LF_ERR_CAPACITY;
  }
  DeviceScope dev(c->device);
  if (!dev.ok()) return LF_ERR_HIP;
  const lf::LayerPtrs p = layer_ptrs(c, layer);
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t* fh = c->fill_host.data() + static_cast<size_t>(layer) * c->cfg.batch;
  // Only the sequences being filled are launched, up to kFillSeqPerLaunch at
  // a time.
  int32_t seqs[lf::kFillSeqPerLaunch], lens[lf::kFillSeqPerLaunch];
  int32_t count = 0;
  for (int32_t b = 0; b <= c->cfg.batch; ++b) {
    if (count == lf::kFillSeqPerLaunch || (b == c->cfg.batch && count > 0)) {
      if (lf::launch_fill(c->geo, p, k, v, seqs, lens, count, n_max, st) != hipSuccess)
        return LF_ERR_HIP;
      count = 0;
    }
    if (b < c->cfg.batch && n_per_seq[b] >= 0) {
      seqs[count] = b;
      lens[count] = n_per_seq[b];
      ++count;
    }
  }
  for (int32_t b = 0; b < c->cfg.batch; ++b)
    if (n_per_seq[b] >= 0) fh[b] = n_per_seq[b];
  if (write_order(c, layer, st) != hipSuccess) return LF_ERR_HIP;
  return LF_OK;
}

lf_status lf_seq_reset(lf_cache* c, const int32_t* seqs, int32_t count, void* stream) {
  if (!c || count < 0 || (count > 0 && !seqs)) return LF_ERR_INVALID_ARG;
  for (int32_t i = 0; i < count; ++i)
    if (seqs[i] < 0 || seqs[i] >= c->cfg.batch) return LF_ERR_INVALID_ARG;
  if (count == 0) return LF_OK;
  DeviceScope dev(c->device);
  if (!dev.ok()) return LF_ERR_HIP;
  hipStream_t st = static_cast<hipStream_t>(stream);
  for (int32_t i0 = 0; i0 < count; i0 += lf::kFillSeqPerLaunch) {
    const int32_t n = std::min<int32_t>(lf::kFillSeqPerLaunch, count - i0);
    if (lf::launch_seq_reset(c->geo, c->cfg.num_layers, c->fill, c->victim, seqs + i0, n, st) !=
        hipSuccess)
      return LF_ERR_HIP;
  }
  for (int32_t l = 0; l < c->cfg.num_layers; ++l)
    for (int32_t i = 0; i < count; ++i)
      c->fill_host[static_cast<size_t>(l) * c->cfg.batch + seqs[i]] = 0;
  for (int32_t l = 0; l < c->cfg.num_layers; ++l)
    if (write_order(c, l, st) != hipSuccess) return LF_ERR_HIP;
  return LF_OK;
}

lf_status lf_decode_step(lf_cache* c, int32_t layer, const void* q, const void* k_new,
                         const void* v_new, void* out, int32_t* evicted_slot, void* stream) {
  return decode_step(c, layer, q, k_new, v_new, out, evicted_slot, stream, false);
}

lf_status lf_decode_step_noalloc(lf_cache* c, int32_t layer, const void* q, const void* k_new,
                                 const void* v_new, void* out, int32_t* evicted_slot, void* stream) {
  return decode_step(c, layer, q, k_new, v_new, out, evicted_slot, stream, true);
}

lf_status lf_probe_stream_plan(int64_t pairs, int32_t n_max, int32_t cus, int32_t resident4,
                               int32_t fits8, int32_t rows, int32_t stride, int32_t forced_stream,
                               int32_t forced_grid, int32_t* plan) {
  if (!plan || pairs < 1 || n_max < 0 || cus < 1 || resident4 < 1 || rows < 0 || stride < 0)
    return LF_ERR_INVALID_ARG;
  const StreamInputs in{pairs, n_max, cus, resident4, fits8 != 0, rows, stride, forced_stream,
                        forced_grid, 0};
  bool eight = false;
  const lf::GridPlan g = stream_plan(in, &eight);
  const int32_t out[8] = {g.grid, g.sk_first, g.sk_pairs, g.sk_tiles, g.sk_q, g.sk_wgs, g.sk_stride,
                          eight ? 8 : 4};
  std::memcpy(plan, out, sizeof(out));
  return LF_OK;
}

lf_status lf_probe_decode_timing(lf_cache* c, int32_t layer, const void* q, const void* k_new,
                                 const void* v_new, void* out, int32_t* evicted_slot,
                                 uint64_t* records, int64_t capacity, int32_t* workgroups,
                                 void* stream) {
  const Timing t{records, capacity, workgroups, nullptr};
  return decode_step(c, layer, q, k_new, v_new, out, evicted_slot, stream, false, &t);
}

lf_status lf_probe_decode_phases(lf_cache* c, int32_t layer, const void* q, const void* k_new,
                                 const void* v_new, void* out, int32_t* evicted_slot,
                                 uint64_t* records, uint64_t* phases, int64_t capacity,
                                 int32_t* workgroups, void* stream) {
  if (!lf::kPhaseStamps) return LF_ERR_UNSUPPORTED;  // the measurement build records phases
  if (!phases) return LF_ERR_INVALID_ARG;
  const Timing t{records, capacity, workgroups, phases};
  return decode_step(c, layer, q, k_new, v_new, out, evicted_slot, stream, false, &t);
}

}  // extern "C"
