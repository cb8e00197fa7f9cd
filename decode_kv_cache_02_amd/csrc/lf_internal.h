// Internal interface between the host runtime (lf_runtime.cpp) and the
// gfx950 kernels (lf_kernels.hip). Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lf {

// Shapes and parameters of one cache, fixed at create time.
struct Geometry {
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;        // num_q_heads / num_kv_heads
  int32_t head_dim;
  int32_t budget;       // EVICT: slots; FULL: capacity
  int32_t sink_size;
  int32_t slots_pad;    // budget rounded up to 64
  int32_t dtype;        // lf_dtype
  int32_t mode;         // lf_mode
  int32_t order;        // lf_order
  int32_t scope;        // lf_scope
  int32_t norm;         // lf_norm
  int64_t pair_elems;   // slots_pad * head_dim
  float scale;          // tau
};

// Device regions of one layer.
struct LayerPtrs {
  void* k;
  void* v;
  float* vnorm;
  int32_t* fill;
  int32_t* victim;    // deferred order: next victim per pair, -1 = none
  // FULL mode: the sequences of the layer in launch order (longest first),
  // [batch]; the decode launch maps its workgroups through it.
  int32_t* order;
};

// Split-K workspace of one layer launch: per (pair, split) the partial
// softmax state, per pair the raw logits of a full cache and an arrival
// counter (zero between launches).
struct SplitWork {
  float* part;        // [pairs][max_splits][split_part_floats]
  float* logit;       // [pairs][slots_pad][group]
  int32_t* arrive;    // [pairs]
  // One victim per sequence: every pair's score vector and, per sequence, an
  // arrival counter of its KV heads (zero between launches).
  float* score;       // [batch][num_kv_heads][slots_pad]
  float* new_norm;    // [batch][num_kv_heads]: ||v_new|| of every head
  int32_t* seq_arrive;  // [batch]
  // Optional timing records, one per workgroup of the launch (null: none):
  // [start, end, XCC id | hardware id << 32, workgroup index], uint64 each;
  // optional phase stamps, eight uint64 per workgroup (lf_decode.h).
  uint64_t* wg_clock = nullptr;
  uint64_t* wg_phase = nullptr;
};

// The measurement build (compiled with LF_PHASE_STAMPS=1, liblongflow_phases.so)
// records when each phase of a decode step ends (lf_probe_decode_phases);
// the library itself leaves those stamps out.
#ifndef LF_PHASE_STAMPS
#define LF_PHASE_STAMPS 0
#endif
constexpr bool kPhaseStamps = LF_PHASE_STAMPS != 0;

constexpr int kMaxSplits = 16;
// Split-K workspace sizing (no device query, so that lf_cache_bytes works
// without a GPU): layers with fewer than kSplitPairsBelow pairs get room for
// kSplitGridTarget / pairs splits (at most kMaxSplits), which covers the
// launch plan's CUs / pairs on devices of up to kSplitGridTarget CUs.
constexpr int kSplitGridTarget = 512;
constexpr int kSplitPairsBelow = 256;
constexpr int kMinSplitSlots = 256;   // fewer slots per split are not worth a split
// Stream launches (GridPlan): the evicting main path gets workspace rows
// (kMaxSplits parts each, at most kStreamRows) for the pairs a stream launch
// would cut on a device of kStreamCusRef compute units (MI355X) with one or
// two resident 4-wave workgroups per compute unit, decided from the
// configuration alone so that lf_cache_bytes needs no device; on another
// device a launch streams only if its cut pairs fit. A workgroup's share is
// at least kStreamMinTiles tiles.
constexpr int kStreamRows = 512;
constexpr int kStreamCusRef = 256;
constexpr int kStreamMinTiles = 16;
// Launches whose workgroups stream at most this many slots use the
// interleaved loop (K and V of each tile together, both streams in flight
// from the start); longer streams use the phased loop (K, then V).
constexpr int kInterleaveSlots = 1024;

// Dynamic LDS bytes the decode kernel needs for this geometry and loop kind
// (ilv: interleaved), or 0 if the combination (dtype, head_dim, group,
// slots) is not built. decode_score_lds_bytes is the part the phased loop
// keeps for the scores of one victim per sequence.
size_t decode_lds_bytes(const Geometry& g, bool ilv);
size_t decode_split_lds_bytes(const Geometry& g, int splits, bool ilv);
size_t decode_score_lds_bytes(const Geometry& g);
size_t split_part_floats(const Geometry& g);

// LDS bytes one workgroup may use on the current device.
size_t device_lds_limit();

// How a launch of the evicting main path (4 waves, no split, no variant)
// spreads its pairs over workgroups; the runtime plans it. grid = 0: one
// workgroup per pair. grid > 0: decode_kernel_stream with `grid` workgroups:
// whole pairs [0, sk_first) taken in turn, then pairs [sk_first, sk_first +
// sk_pairs) as one run of sk_pairs * sk_tiles tiles dealt out sk_q at a time
// to workgroups 0 .. sk_wgs - 1, a pair cut between workgroups combining its
// parts through workspace rows of sk_stride partials (row = pair - sk_first).
struct GridPlan {
  int grid = 0;
  int sk_first = 0;
  int sk_pairs = 0;
  int sk_tiles = 0;
  int sk_q = 0;
  int sk_wgs = 0;
  int sk_stride = 0;
};

// splits == 1: one workgroup per pair, or the stream launch of `plan`.
// splits > 1: split-K over `splits` workgroups per pair (W must then hold
// room for that many). waves: 4 or 8 waves of 64 lanes per workgroup (8 when
// one workgroup per CU is all the launch has). ilv: the interleaved loop
// instead of the phased one.
hipError_t launch_decode(const Geometry& g, const LayerPtrs& L, const SplitWork& W, int splits, int waves,
                         bool ilv, const GridPlan& plan, const void* q, const void* k_new,
                         const void* v_new, void* out, int32_t* evicted, hipStream_t stream);
#define LF_DECLARE_DECODE_UNIT(NAME)                                                          \
  hipError_t NAME(const Geometry& g, const LayerPtrs& L, const SplitWork& W, int splits,    \
                  const GridPlan& plan, const void* q, const void* k_new, const void* v_new, \
                  void* out, int32_t* evicted, hipStream_t stream);
LF_DECLARE_DECODE_UNIT(launch_decode_w4)   // lf_decode_w4.hip: 4 waves, phased
LF_DECLARE_DECODE_UNIT(launch_decode_w8)   // lf_decode_w8.hip: 8 waves, phased
LF_DECLARE_DECODE_UNIT(launch_decode_w4i)  // lf_decode_w4i.hip: 4 waves, interleaved
LF_DECLARE_DECODE_UNIT(launch_decode_w8i)  // lf_decode_w8i.hip: 8 waves, interleaved
#undef LF_DECLARE_DECODE_UNIT

// Static LDS of a decode workgroup of `waves` waves (per-wave output
// partials and reduction scratch), an upper bound.
size_t decode_static_lds_bytes(const Geometry& g, int waves);

// Copies rows [0, n_i) of sequence seq_host[i] into slots 0..n_i-1 of each
// of its pairs, for `count` listed sequences (host arrays); slots past n_i
// keep what they held.
hipError_t launch_fill(const Geometry& g, const LayerPtrs& L, const void* k,
                       const void* v, const int32_t* seq_host, const int32_t* n_host,
                       int32_t count, int32_t n_max, hipStream_t stream);

// Drops every layer's pairs of the `count` sequences in seqs_host to 0 tokens
// with no pending victim.
hipError_t launch_seq_reset(const Geometry& g, int32_t num_layers, int32_t* fill, int32_t* victim,
                            const int32_t* seqs_host, int32_t count, hipStream_t stream);

constexpr int kFillSeqPerLaunch = 256;

// Writes the launch order of `count` sequences, order[first + i] = seq[i]
// (host array), into one layer's order array.
constexpr int kOrderPerLaunch = 512;
hipError_t launch_set_order(int32_t* order, const int32_t* seq_host, int32_t first, int32_t count,
                            hipStream_t stream);

// Static scratch of lf_decode_step_noalloc (lf_scratch.hip): one device array
// per GPU. The first kScratchCounterBytes hold arrival counters only (zero
// between launches): split-K counters at word 0 + pair, per-sequence counters
// at word kScratchSeqCounterWord + sequence. The rest holds the workspace
// of one launch.
constexpr size_t kScratchBytes = size_t{64} << 20;
constexpr size_t kScratchCounterBytes = size_t{64} << 10;
constexpr int32_t kScratchSeqCounterWord = 8192;
// Looks up the array's device address on `device` (which must be current)
// and clears its counters, once per device. Never called under capture.
hipError_t scratch_setup(int device);
// The address kept by scratch_setup, or null before it has run.
void* scratch_ptr(int device);

}  // namespace lf
