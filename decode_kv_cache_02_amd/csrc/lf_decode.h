#pragma once
// gfx950 (MI355X) decode kernel of the LongFlow fused decode + score + evict
// step, as a template shared by the translation units that instantiate it
// (one per workgroup size and loop) and the device helpers the fill kernel
// also uses.
//
// The step is defined on the LongFlow pages: attention weights and output
// (LongFlow Guide, §Mathematical Derivation of the LongFlow Score, alpha and
// o_t equations), the score alpha_i * ||v_i||_1 (same section, c_{t,i} and
// Score equations; gist.science summary of arXiv 2603.11504, §2.1) and the
// static buffer with argmin eviction and in-place overwrite (LongFlow Guide,
// §Static Memory Pre-Allocation and In-Place Eviction). The pages' own kernel
// (LongFlow Guide, §Fused High-Performance Triton Attention Kernel; summary
// §2.3) is a single pass that scores tokens from tiles already on chip; the
// design below keeps that property for gfx950:
//
//   one workgroup = one pair (sequence, KV head), 4 or 8 waves of 64 lanes
//   (split-K: a contiguous range of the pair's 16-slot tiles). K is stored
//   in MFMA operand order, so 16-byte loads land straight in the B operand
//   of v_mfma_f32_16x16x32_bf16 (16x16x4 f32 for float32 caches); the query
//   group is replicated over the 16 A rows, so each lane holds all G logits
//   of one slot. The raw logits of the whole range stay in LDS.
//   Phased loop (long streams)
//            K stream: logits to LDS, two register sets in flight.
//            Transition: max M and sum L (the new token included), p in
//            place, the score and its argmin, while the first V rows are in
//            flight. V stream: o += p v, two register sets in flight.
//   Interleaved loop (streams of up to 1024 slots per workgroup)
//            each wave takes every WAVES-th tile and streams its K and the V
//            rows of the same slots together, two tiles in flight, with its
//            own online softmax (p staged in a per-wave strip of LDS). After
//            one barrier: M, L and each wave's rescaling factor in a fixed
//            order, the output, then the score from the raw logits.
//   Score    score_i = ||v_i|| * sum_g exp2(s_{g,i} - M_g)/L_g from the raw
//            logits and the float32 sidecar; (score, slot) argmin through DPP
//            and LDS, lowest slot on ties; the new token's K, V and ||v|| are
//            written in place.
//   Split-K  every split publishes its (m, l, o) and, when scoring, its raw
//            logits; the last split to arrive combines, scores and writes.
//            No workgroup waits for another.
//   VAR      the engine's deferred order and one victim per sequence, as
//            run-time flags of separate instances (the main instance carries
//            neither).
//
// Every cached byte is read once: the score needs no second pass over HBM
// because the raw logits stay in LDS until M and L are known.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lf_internal.h"

namespace lf {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kStream = 3;                          // cache policy: non-temporal (nt) + sc0
constexpr size_t kEvictLdsCap = 144 * 1024;        // logits of one pair; the rest is static LDS
constexpr size_t kFullChunkSlots = 2048;            // FULL mode, phased loop: slots per LDS chunk
constexpr float kSlack = 32.0f;                     // online softmax: rescale when a logit exceeds
                                                    // the reference maximum by more (log2 units)
constexpr float kNoMax = -1.0e30f;                  // reference maximum before any live slot
constexpr float kLog2e = 1.4426950408889634f;

// Storage types: float32 is `float`, bfloat16 is its 16-bit pattern.
template <typename T> struct Elem;
template <> struct Elem<float> { static constexpr int kBytes = 4; };
template <> struct Elem<uint16_t> { static constexpr int kBytes = 2; };

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

__device__ __forceinline__ void from_f32(float x, float* dst) { *dst = x; }
__device__ __forceinline__ void from_f32(float x, uint16_t* dst) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) {
    *dst = 0x7fc0;  // quiet NaN
    return;
  }
  u += 0x7fffu + ((u >> 16) & 1u);  // round to nearest, ties to even
  *dst = static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ u32x4_t load16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}
__device__ __forceinline__ void store16(void* p, u32x4_t x) {
  *reinterpret_cast<u32x4_t*>(p) = x;
}

// Raw buffer resource over `bytes` bytes at `base`: 32-bit offsets, and any
// 16-byte load that starts at or beyond `bytes` returns zeros.
constexpr int kRsrcWord3 = 0x00020000;  // raw, 32-bit data format
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), kRsrcWord3);
}
// POLICY is the instruction's cache-policy field; kStream marks the K/V rows
// as non-temporal (each is read once per step, and a step's rows do not fit
// in the caches).
template <int POLICY = 0>
__device__ __forceinline__ u32x4_t bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, POLICY);
}

// K is stored in 16-slot tiles of 1 KB blocks: within tile t (16 rows of D
// elements), block c holds, at byte 64 * r + 16 * j, the 16 bytes of slot
// 16t + r that cover 16-byte chunk 4c + j of the row. One wave-wide 16-byte
// load per block reads the block's 1 KB, and lane l takes byte
// k_lane_offset(l) = 64 * (l % 16) + 16 * (l / 16), which lands the block
// in MFMA B-operand order (slot l % 16, k-group l / 16). A slot's row is 4
// contiguous 64-byte pieces per 4 KB tile (D = 128, bf16), so replacing it
// in place touches 4 places, not one 16-byte chunk in each of 16 cache
// lines. V stays row-major.
template <int ROW_BYTES>
__device__ __forceinline__ uint32_t k_chunk_offset(int slot, int chunk) {
  return static_cast<uint32_t>(slot >> 4) * (16u * ROW_BYTES) +
         static_cast<uint32_t>(chunk >> 2) * 1024u +
         static_cast<uint32_t>(slot & 15) * 64u + static_cast<uint32_t>(chunk & 3) * 16u;
}
__device__ __forceinline__ uint32_t k_lane_offset(int lane) {
  return 64u * static_cast<uint32_t>(lane & 15) + 16u * static_cast<uint32_t>(lane >> 4);
}

// G consecutive floats of LDS as one vector access.
template <int G> struct PVec;
template <> struct PVec<1> { typedef float type; };
template <> struct PVec<2> { typedef float type __attribute__((ext_vector_type(2))); };
template <> struct PVec<4> { typedef float type __attribute__((ext_vector_type(4))); };

template <int G>
__device__ __forceinline__ void lds_get(const float* base, int i, float (&x)[G]) {
  const typename PVec<G>::type v = *reinterpret_cast<const typename PVec<G>::type*>(base + i * G);
  if constexpr (G == 1) {
    x[0] = v;
  } else {
#pragma unroll
    for (int g = 0; g < G; ++g) x[g] = v[g];
  }
}
template <int G>
__device__ __forceinline__ void lds_put(float* base, int i, const float (&x)[G]) {
  typename PVec<G>::type v;
  if constexpr (G == 1) {
    v = x[0];
  } else {
#pragma unroll
    for (int g = 0; g < G; ++g) v[g] = x[g];
  }
  *reinterpret_cast<typename PVec<G>::type*>(base + i * G) = v;
}

// 16 loaded bytes -> float32 values.
__device__ __forceinline__ void unpack16(u32x4_t w, float (&x)[8], uint16_t) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack16(u32x4_t w, float (&x)[4], float) {
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(w[i]);
}

// One 16-byte chunk of a query row times the matching chunk of 16 key rows.
// A operand = query (row i of the 16x16 tile = query head i % G),
// B operand = keys (column j = slot j of the tile).
__device__ __forceinline__ f32x4_t mfma_chunk(u32x4_t qa, u32x4_t kb, f32x4_t acc, uint16_t) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qa),
                                                 __builtin_bit_cast(bf16x8_t, kb), acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_chunk(u32x4_t qa, u32x4_t kb, f32x4_t acc, float) {
#pragma unroll
  for (int m = 0; m < 4; ++m)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(qa[m]), __uint_as_float(kb[m]),
                                               acc, 0, 0, 0);
  return acc;
}

// Wave-wide reductions: DPP butterflies inside each row of 16 lanes (xor 1,
// xor 2, rotate 4, rotate 8), then the four row results combined from lanes
// 0, 16, 32 and 48 in that order. The result is the same in every lane.
constexpr int kDppXor1 = 0xB1;   // quad_perm(1,0,3,2)
constexpr int kDppXor2 = 0x4E;   // quad_perm(2,3,0,1)
constexpr int kDppRor4 = 0x124;  // row_ror:4
constexpr int kDppRor8 = 0x128;  // row_ror:8

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(x), CTRL, 0xF, 0xF, false));
}
// Ordering point for lanes of one wave that exchange values through LDS
// without a workgroup barrier. The hardware runs one wave's LDS operations in
// issue order, but the compiler reasons per lane: a lane that does not take
// part in a guarded write could otherwise have its read of the same strip
// moved ahead of the write. Wavefront-scope release and acquire fences
// around a wave barrier keep every lane's accesses on their side of it.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float lane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_f<kDppXor1>(x);
  x += dpp_f<kDppXor2>(x);
  x += dpp_f<kDppRor4>(x);
  x += dpp_f<kDppRor8>(x);
  return (lane_f(x, 0) + lane_f(x, 16)) + (lane_f(x, 32) + lane_f(x, 48));
}
// Sum over each row of 16 lanes (the same DPP butterflies as wave_sum); every
// lane of a row ends with its row's sum.
__device__ __forceinline__ float row_sum(float x) {
  x += dpp_f<kDppXor1>(x);
  x += dpp_f<kDppXor2>(x);
  x += dpp_f<kDppRor4>(x);
  x += dpp_f<kDppRor8>(x);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f<kDppXor1>(x));
  x = fmaxf(x, dpp_f<kDppXor2>(x));
  x = fmaxf(x, dpp_f<kDppRor4>(x));
  x = fmaxf(x, dpp_f<kDppRor8>(x));
  return fmaxf(fmaxf(lane_f(x, 0), lane_f(x, 16)), fmaxf(lane_f(x, 32), lane_f(x, 48)));
}

// Lexicographic (score, slot) minimum over the wave. Scores are >= 0, so
// their float bits order like unsigned integers and (bits, slot) compares as
// one 64-bit key: the smallest score wins, then the lowest slot.
__device__ __forceinline__ void key_min(uint32_t& hi, uint32_t& lo, uint32_t h2, uint32_t l2) {
  if (h2 < hi || (h2 == hi && l2 < lo)) {
    hi = h2;
    lo = l2;
  }
}
template <int CTRL>
__device__ __forceinline__ void key_min_dpp(uint32_t& hi, uint32_t& lo) {
  const uint32_t h2 = dpp_u<CTRL>(hi);
  const uint32_t l2 = dpp_u<CTRL>(lo);
  key_min(hi, lo, h2, l2);
}
__device__ __forceinline__ void wave_argmin(float& score, int& slot) {
  uint32_t hi = __float_as_uint(score);
  uint32_t lo = static_cast<uint32_t>(slot);
  key_min_dpp<kDppXor1>(hi, lo);
  key_min_dpp<kDppXor2>(hi, lo);
  key_min_dpp<kDppRor4>(hi, lo);
  key_min_dpp<kDppRor8>(hi, lo);
  uint32_t bh = __builtin_amdgcn_readlane(hi, 0), bl = __builtin_amdgcn_readlane(lo, 0);
#pragma unroll
  for (int r = 16; r < kWave; r += 16)
    key_min(bh, bl, __builtin_amdgcn_readlane(hi, r), __builtin_amdgcn_readlane(lo, r));
  score = __uint_as_float(bh);
  slot = static_cast<int>(bl);
}

// ||row||_1 (or ||row||_2 when l2) in float32 in one fixed order, evaluated
// by a whole wave from the row's elements lane + k * 64 (already loaded); the
// result is lane 0's. The fill and the decode kernels both use this routine,
// so equal stored rows always get bit-equal sidecar values.
template <typename T, int D>
__device__ __forceinline__ float wave_norm_vals(const T (&v)[D / kWave], bool l2) {
  float x = 0.0f;
#pragma unroll
  for (int k = 0; k < D / kWave; ++k) {
    const float f = to_f32(v[k]);
    x = l2 ? fmaf(f, f, x) : x + fabsf(f);
  }
  const float s = wave_sum(x);
  return l2 ? sqrtf(s) : s;
}
template <typename T, int D>
__device__ __forceinline__ float wave_norm(const T* row, int lane, bool l2) {
  T v[D / kWave];
#pragma unroll
  for (int k = 0; k < D / kWave; ++k) v[k] = row[lane + k * kWave];
  return wave_norm_vals<T, D>(v, l2);
}

struct DecodeParams {
  const void* q;
  const void* k_new;
  const void* v_new;
  void* out;
  int32_t* evicted;
  const void* kc;
  const void* vc;
  void* kc_w;
  void* vc_w;
  float* vnorm;         // ||v||_1 (or ||v||_2) sidecar
  int32_t* fill;
  int32_t* victim;      // deferred order: next victim per pair, -1 = none
  int64_t pair_elems;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t budget;
  int32_t sink;
  int32_t chunk;        // phased loop: slots per LDS-resident chunk (EVICT: the whole split)
  float scale_log2;     // tau * log2(e)
  int32_t deferred;     // 1: write into the previous victim, then choose the next
  int32_t shared;       // 1: one victim per sequence (scores summed over KV heads)
  int32_t norm_l2;      // 1: the sidecar holds ||v||_2
  // Split-K across workgroups (SPLIT kernels only).
  int32_t pairs;        // pairs of the layer
  int32_t splits;       // workgroups per pair
  float* ws_part;       // [pairs][splits][2G + G*D]: m, l, unnormalised output
  float* ws_logit;      // [pairs][slots_pad][G]: raw logits (cache full only)
  int32_t* arrive;      // [pairs]: arrivals, back to 0 after every launch
  // One victim per sequence.
  float* ws_score;      // [batch][num_kv_heads][slots_pad]: every head's score vector
  float* ws_nnorm;      // [batch][num_kv_heads]: every head's ||v_new||
  int32_t* seq_arrive;  // [batch]: KV heads done, back to 0 after every launch
  uint64_t* wg_clock;   // optional: per-workgroup timing records (null: none)
  uint64_t* wg_phase;   // optional: per-workgroup phase stamps [workgroups][8] (null: none)
  const int32_t* order; // FULL mode: sequences in launch order, longest first
  // Stream launch (decode_kernel_stream): pairs [0, sk_first) whole, taken in
  // turn; pairs [sk_first, sk_first + sk_pairs) as one run of sk_pairs *
  // sk_tiles tiles dealt out sk_q at a time to workgroups 0 .. sk_wgs - 1.
  int32_t sk_first;
  int32_t sk_pairs;
  int32_t sk_tiles;     // tiles per pair (of the longest pair)
  int32_t sk_q;         // tiles per workgroup
  int32_t sk_wgs;
  int32_t sk_stride;    // partials per workspace row
};

// One part of a pair in a split launch: which pair, which of its parts, the
// tiles it streams, and the row of the split workspace (partials, raw
// logits, arrival counter) that the pair's parts share.
struct Part {
  int pair;    // the pair, in launch order
  int index;   // 0 .. count - 1
  int count;   // parts of the pair
  int row;     // workspace row
  int stride;  // partials per workspace row
  int t0, t1;  // tiles [t0, t1) of the pair; t0 < 0: part `index` of `count` equal ones
};

// hwreg encodings for s_getreg: XCC_ID (the accelerator complex die a
// workgroup runs on) and HW_ID (its SE, SH, CU, SIMD and wave slot).
constexpr int kHwRegXccId = (15 << 11) | 20;
constexpr int kHwRegHwId = (31 << 11) | 4;

// Timing record of one workgroup, written by thread 0 when it returns: start
// and end of thread 0 on the device's constant 100 MHz clock, where it ran,
// and the workgroup index. Measurement only; a null record costs one
// uniform branch at entry and at return.
struct ClockRecord {
  uint64_t* rec;
  uint64_t start;
  __device__ __forceinline__ ~ClockRecord() {
    if (rec) {
      rec[0] = start;
      rec[1] = __builtin_amdgcn_s_memrealtime();
      rec[2] = static_cast<uint64_t>(__builtin_amdgcn_s_getreg(kHwRegXccId)) |
               (static_cast<uint64_t>(__builtin_amdgcn_s_getreg(kHwRegHwId)) << 32);
      rec[3] = blockIdx.x;
    }
  }
};

// Phase stamps: the constant clock at the end of phases 1..8 of the
// workgroup's last unit (0: not reached), written by thread 0. 1: the
// interleaved loop's first tile processed, or the phased loop's K stream
// done; 2: the stream done; 3: a split's partial state published and
// drained; 4: its ticket back; 5: the last split has every split's (m, l)
// and the pair's max and sum; 6: the last split's score done; 7: the
// in-place write reached. Only the measurement build (kPhaseStamps)
// compiles the stamps in, and only into bfloat16 instances (the float32
// ones have no registers to spare).
template <typename T>
__device__ __forceinline__ void phase_stamp(const DecodeParams& P, int tid, int k) {
  if constexpr (kPhaseStamps && sizeof(T) == 2) {
    if (P.wg_phase && tid == 0) P.wg_phase[8 * static_cast<size_t>(blockIdx.x) + k - 1] = __builtin_amdgcn_s_memrealtime();
  }
}

// Cross-workgroup data of a split launch goes through relaxed agent-scope
// atomic accesses: each is coherent across the XCDs on its own, so no
// whole-cache writeback or invalidate is needed. The writer drains its
// stores before it takes its ticket, and the last split reads only after
// its ticket says every other split has arrived. tests/test_asm_ordering.py
// checks that order on every path of every built kernel.
__device__ __forceinline__ void ws_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ws_load(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void drain_stores() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}
// s_waitcnt vmcnt(0) as an instruction the compiler's own wait placement
// sees (expcnt and lgkmcnt fields at their maxima, so no wait on those):
// after it, no earlier load counts as outstanding, so later stores of
// long-loaded values need no wait behind stores issued in between.
__device__ __forceinline__ void settle_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// The G logits of one slot as one buffer access with the device-scope cache
// policy (the sc1 bit, as the relaxed agent-scope atomics above use).
constexpr int kDeviceScope = 16;
template <int G>
__device__ __forceinline__ void ws_store_g(__amdgpu_buffer_rsrc_t r, uint32_t off, const float (&x)[G]) {
  if constexpr (G == 4) {
    u32x4_t v = {__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                 __float_as_uint(x[3])};
    __builtin_amdgcn_raw_buffer_store_b128(v, r, static_cast<int>(off), 0, kDeviceScope);
  } else if constexpr (G == 2) {
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    u32x2_t v = {__float_as_uint(x[0]), __float_as_uint(x[1])};
    __builtin_amdgcn_raw_buffer_store_b64(v, r, static_cast<int>(off), 0, kDeviceScope);
  } else {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x[0]), r, static_cast<int>(off), 0,
                                          kDeviceScope);
  }
}
template <int G>
__device__ __forceinline__ void ws_load_g(__amdgpu_buffer_rsrc_t r, uint32_t off, float (&x)[G]) {
  if constexpr (G == 4) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, kDeviceScope);
#pragma unroll
    for (int g = 0; g < 4; ++g) x[g] = __uint_as_float(v[g]);
  } else if constexpr (G == 2) {
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, static_cast<int>(off), 0, kDeviceScope);
    x[0] = __uint_as_float(v[0]);
    x[1] = __uint_as_float(v[1]);
  } else {
    x[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(off), 0, kDeviceScope));
  }
}

/*
 * One decode step of one unit of work, by the whole workgroup (thread `tid`).
 *   SPLIT = false: a unit is a pair (unit = pair, in launch order).
 *   SPLIT = true : a unit is one part of a pair (`seg`), a contiguous range
 *                  of 16-slot tiles. Each
 *                  publishes its partial softmax state (m, l, output) and,
 *                  when the cache is full, its raw logits; the last split to
 *                  arrive combines the partials, scores every slot against
 *                  the global max and sum, takes the argmin and writes the
 *                  output and the new token. No workgroup ever waits.
 *   VAR = true: the deferred order and one victim per sequence are available
 *               (runtime flags); false compiles them out of the main path.
 *   ILV = true: the interleaved loop (each wave streams the K and the V of
 *               the same tiles together, UA tiles per set, two sets in
 *               flight); false: the phased loop (all K, then all V, UA K
 *               tiles or UB V row loads per set).
 */
template <typename T, int D, int G, bool EVICT, int WAVES, int UA, int UB, int POLICY, bool SPLIT,
          bool VAR, bool ILV>
__device__ __forceinline__ void decode_unit(const DecodeParams& P, const int unit, const int tid,
                                            const Part& seg) {
  constexpr int kBytes = Elem<T>::kBytes;
  constexpr int NT = WAVES * kWave;
  constexpr int kChunks = D * kBytes / 64;  // 16-byte K loads per lane per 16-slot tile
  constexpr int EPL = 16 / kBytes;          // elements per 16-byte load
  constexpr int LPS = D / EPL;              // lanes per V row
  constexpr int SPI = kWave / LPS;          // V rows per wave-wide load
  constexpr uint32_t kRowBytes = D * kBytes;
  // sidecar loads in flight per thread: the first batch covers NT * kScoreBatch
  // slots (4096 for either workgroup size); later batches load in the loop
  constexpr int kScoreBatch = WAVES >= 8 ? 8 : 16;
  constexpr int kRowLoads = D * kBytes / 16;
  constexpr int kVLoads = 16 / SPI;         // wave-wide V loads per 16-slot tile (= kChunks)
  static_assert(G == 1 || G == 2 || G == 4, "group width");
  static_assert(LPS <= kWave && SPI * LPS == kWave, "row split");
  static_assert(G <= WAVES, "one wave per query head of the group for the new token");

  extern __shared__ __attribute__((aligned(16))) float lds[];  // EVICT: [hi - lo][G] raw logits
  __shared__ float sh_red[WAVES][G][D];     // per-wave output partials
  __shared__ __attribute__((aligned(16))) float sh_pst[WAVES][16 * G];  // per-wave p of one tile
  __shared__ float sh_part[WAVES][G];       // per-wave reference maximum
  __shared__ float sh_part2[WAVES][G];      // per-wave sum of p
  __shared__ float sh_snew[G];
  __shared__ float sh_vn_new;
  __shared__ float sh_best_score[WAVES];
  __shared__ int sh_best_slot[WAVES];
  __shared__ float sh_gm[G];                // last split: the pair's max and sum
  __shared__ float sh_gl[G];
  __shared__ float sh_fac[kMaxSplits][G];  // last split: exp2(m_split - M) per split
  __shared__ int sh_ticket;
  (void)sh_gm;
  (void)sh_gl;
  (void)sh_fac;
  (void)sh_ticket;

  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  // Unit -> (sequence b, KV head h). FULL mode dispatches the sequences
  // longest first (P.order); the evicting cache keeps index order.
  const int slot_in_launch = SPLIT ? seg.pair : unit;
  const int split = SPLIT ? seg.index : 0;
  const int h = slot_in_launch % P.num_kv_heads;
  int b = slot_in_launch / P.num_kv_heads;
  if constexpr (!EVICT) {
    if (P.order) b = min(max(P.order[b], 0), P.pairs / P.num_kv_heads - 1);
  }
  const int pair = b * P.num_kv_heads + h;
  const int64_t slots_pad = P.pair_elems / D;

  const T* K = static_cast<const T*>(P.kc) + pair * P.pair_elems;
  const T* V = static_cast<const T*>(P.vc) + pair * P.pair_elems;
  const T* qg = static_cast<const T*>(P.q) + (static_cast<int64_t>(b) * P.num_q_heads + h * G) * D;
  const T* kn = static_cast<const T*>(P.k_new) + static_cast<int64_t>(pair) * D;
  const T* vn = static_cast<const T*>(P.v_new) + static_cast<int64_t>(pair) * D;
  // The host keeps 0 <= n <= budget (and n < budget in FULL mode); clamping
  // keeps every access inside the pair's region even if that were broken.
  const int n = min(max(P.fill[pair], 0), P.budget);
  constexpr uint32_t kTileBytes = 16 * kRowBytes;

  // This workgroup's slots: [lo, hi), whole 16-slot tiles.
  int lo = 0, hi = n;
  if (SPLIT) {
    const int tiles = (n + 15) >> 4;
    int tb, te;
    if (seg.t0 >= 0) {
      tb = min(seg.t0, tiles);
      te = min(seg.t1, tiles);
    } else {
      const int per = (tiles + seg.count - 1) / seg.count;
      tb = min(split * per, tiles);
      te = min(tb + per, tiles);
    }
    lo = tb * 16;
    hi = min(te * 16, n);
  }

  // Lane roles. K: r16 = slot within a 16-slot tile, grp = 16-byte chunk
  // group. V: vcol = first element of the lane's 16 bytes of the row, vsub =
  // which of the SPI rows of a wave-wide load.
  const int r16 = lane & 15;
  const int grp = lane >> 4;
  const int vcol = (lane % LPS) * EPL;
  const int vsub = lane / LPS;

  // What this step does with the new token.
  //   same-step order: below the budget it is appended at slot n; at the
  //     budget the cached slots are scored and the argmin is overwritten.
  //   deferred order: below the budget it is appended; at the budget it
  //     replaces `masked`, the previous step's victim (budget-1 if none),
  //     whose old token then takes no part in the step. The cached slots are
  //     scored whenever the buffer is full after the write, and the argmin
  //     becomes the next victim.
  const bool deferred = VAR && P.deferred;
  const bool shared = VAR && P.shared;
  const bool overwrite = EVICT && n >= P.budget;
  int masked = -1;
  if (EVICT && deferred && overwrite) {
    const int v = P.victim[pair];
    masked = (v >= 0 && v < P.budget) ? v : P.budget - 1;
  }
  const bool scoring = EVICT && (deferred ? n + 1 >= P.budget : overwrite);

  // The new token's logits (wave g < G takes query head g) and ||v_new||
  // (wave 0). Their inputs are requested now and used after the stream, so
  // no wave starts its tiles late; the results are visible after the
  // workgroup's first barrier.
  T nq[D / kWave], nk[D / kWave], nv[D / kWave];
  {
    const int hsel = wave < G ? wave : 0;
#pragma unroll
    for (int k = 0; k < D / kWave; ++k) {
      const int d = lane + k * kWave;
      nq[k] = qg[hsel * D + d];
      nk[k] = kn[d];
      nv[k] = vn[d];
    }
  }
  // What the epilogue reads of the new token, requested now as well: v_new
  // at this thread's output elements (the new token's own term) and, for
  // the threads that store the new row, one 16-byte chunk of k_new or v_new.
  constexpr int kOutPer = (G * D + NT - 1) / NT;  // output elements per thread
  T ov[kOutPer];
#pragma unroll
  for (int j = 0; j < kOutPer; ++j) ov[j] = vn[(tid + j * NT) % D];
  u32x4_t wrow = {0u, 0u, 0u, 0u};
  if (tid < kRowLoads)
    wrow = load16(kn + tid * EPL);
  else if (tid < 2 * kRowLoads)
    wrow = load16(vn + (tid - kRowLoads) * EPL);
  auto new_token = [&]() {
    if (wave < G) {
      float x = 0.0f;
#pragma unroll
      for (int k = 0; k < D / kWave; ++k) x = fmaf(to_f32(nq[k]), to_f32(nk[k]), x);
      x = wave_sum(x);
      if (lane == 0) sh_snew[wave] = x * P.scale_log2;
    }
    if (wave == 0) {
      const float nrm = wave_norm_vals<T, D>(nv, P.norm_l2 != 0);
      if (lane == 0) sh_vn_new = nrm;
    }
  };

  // This pair's output rows [G][D].
  auto out_rows = [&]() {
    return static_cast<T*>(P.out) + (static_cast<int64_t>(b) * P.num_q_heads + h * G) * D;
  };
  float best = INFINITY;  // this thread's (score, slot) minimum
  int best_i = 0x7fffffff;
  constexpr int kPart = 2 * G + G * D;  // split partial: m[G], l[G], o[G][D]
  const int S = SPLIT ? seg.count : 1;  // parts of this pair
  // This pair's row of the split workspace: partials, raw logits, counter.
  const int64_t wsr = SPLIT ? seg.row : pair;
  const int64_t wstride = SPLIT ? seg.stride : 1;
  (void)S;
  (void)wsr;
  (void)wstride;

  if constexpr (ILV) {
    // ======== Interleaved loop: K and V of each tile together ========
    // For short streams (small batches, split-K, small budgets): both
    // streams in flight from the first tile and no barrier until the end.
    // The K tiles and V rows of [lo, hi) are read through descriptors that end
    // at hi (whole tiles for K): the loop always requests the next set, and
    // requests past the end return zeros without moving data, so the
    // compiler's load counting stays exact and both sets stay in flight.
    const int ntiles = (hi - lo + 15) >> 4;
    const __amdgpu_buffer_rsrc_t rK =
        make_rsrc(K, static_cast<uint32_t>((hi + 15) >> 4) * kTileBytes);
    const __amdgpu_buffer_rsrc_t rV = make_rsrc(V, static_cast<uint32_t>(hi) * kRowBytes);
    const uint32_t kbase = static_cast<uint32_t>(lo >> 4) * kTileBytes + k_lane_offset(lane);
    const uint32_t vbase = static_cast<uint32_t>(lo + vsub) * kRowBytes + vcol * kBytes;
    // One set = UA tiles: their K (kChunks loads each) and the V rows of the
    // same slots (kVLoads loads each).
    auto load_set = [&](u32x4_t (&kt)[UA][kChunks], u32x4_t (&vt)[UA][kVLoads], int t0) {
#pragma unroll
      for (int u = 0; u < UA; ++u)
#pragma unroll
        for (int c = 0; c < kChunks; ++c)
          kt[u][c] = bload16<POLICY>(
              rK, kbase + static_cast<uint32_t>(t0 + u) * kTileBytes + 1024u * c);
#pragma unroll
      for (int u = 0; u < UA; ++u)
#pragma unroll
        for (int j = 0; j < kVLoads; ++j)
          vt[u][j] = bload16<POLICY>(
              rV, vbase + static_cast<uint32_t>((t0 + u) * 16 + j * SPI) * kRowBytes);
    };

    // The first set goes out before anything else.
    u32x4_t kr[UA][kChunks], vr[UA][kVLoads];
    load_set(kr, vr, wave * UA);

    // Query operand in the MFMA A layout: lane = row (query head row % G) +
    // 16 * (16-byte chunk group); the same byte offsets as the key loads.
    u32x4_t qa[kChunks];
#pragma unroll
    for (int c = 0; c < kChunks; ++c)
      qa[c] = load16(qg + (r16 % G) * D + (64 * c + 16 * grp) / kBytes);

    // Sidecar of the slots this thread scores (the first kScoreBatch of them),
    // requested now so the score pass finds it in registers.
    const __amdgpu_buffer_rsrc_t rN =
        make_rsrc(P.vnorm + static_cast<int64_t>(pair) * slots_pad, static_cast<uint32_t>(hi) * 4u);
    float vnb[kScoreBatch];
    if (!SPLIT && scoring) {
#pragma unroll
      for (int k = 0; k < kScoreBatch; ++k)
        vnb[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            rN, static_cast<int>((P.sink + tid + k * NT) * 4), 0, 0));
    }

    // ---------------- Stream: K and V of each tile together ----------------
    // Every wave runs its own online softmax over its tiles (t = wave, wave +
    // WAVES, ...). m_w is a reference maximum, raised (with acc and lsum
    // rescaled) only when a logit exceeds it by more than kSlack, so
    // p = exp2(s - m_w) stays below 2^kSlack and float32 sums cannot overflow.
    // Per tile: the MFMA logits (raw values kept in LDS for the score pass
    // when evicting), p for the 16 slots x G heads staged in this wave's strip
    // of LDS, then the V rows of the same slots accumulated against p. Every
    // lane holds all G logits of its slot (the four chunk groups hold copies),
    // so p is split over the lanes: lane (grp, r16) evaluates head grp of slot
    // r16 when grp < G, and keeps the running sum of its head's p.
    const int hg = grp & (G - 1);  // this lane's head in the p and sum work
    float m_w[G], lsum = 0.0f;
    float acc[G][EPL];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m_w[g] = kNoMax;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] = 0.0f;
    }
    float* pst = &sh_pst[wave][0];
    auto process = [&](const u32x4_t (&kt)[UA][kChunks], const u32x4_t (&vt)[UA][kVLoads], int t0) {
#pragma unroll
      for (int u = 0; u < UA; ++u) {
        const int t = t0 + u;
        if (t < ntiles) {
          f32x4_t s4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int c = 0; c < kChunks; ++c) s4 = mfma_chunk(qa[c], kt[u][c], s4, T());
          const int i = t * 16 + r16;  // slot - lo
          const bool live = lo + i < hi && (!VAR || lo + i != masked);
          float s[G];
          bool bump = false;
#pragma unroll
          for (int g = 0; g < G; ++g) {
            s[g] = live ? s4[g] * P.scale_log2 : -INFINITY;
            bump = bump || s[g] > m_w[g] + kSlack;
          }
          if (EVICT && grp == 0) lds_put<G>(lds, i, s);
          if (__builtin_amdgcn_ballot_w64(bump) != 0) {  // wave-uniform
#pragma unroll
            for (int g = 0; g < G; ++g) {
              const float m_new = fmaxf(m_w[g], wave_max(s[g]));
              const float f = __builtin_amdgcn_exp2f(m_w[g] - m_new);
              m_w[g] = m_new;
              if (hg == g) lsum *= f;
#pragma unroll
              for (int e = 0; e < EPL; ++e) acc[g][e] *= f;
            }
          }
          float sg = s[0], mg = m_w[0];
#pragma unroll
          for (int g = 1; g < G; ++g) {
            sg = hg == g ? s[g] : sg;
            mg = hg == g ? m_w[g] : mg;
          }
          const float pv = __builtin_amdgcn_exp2f(sg - mg);  // v_exp_f32; -inf -> 0
          if (grp < G) {
            pst[r16 * G + hg] = pv;
            lsum += pv;
          }
          wave_lds_sync();  // every lane reads the strip after the lanes above wrote it
#pragma unroll
          for (int j = 0; j < kVLoads; ++j) {
            float x[EPL];
            unpack16(vt[u][j], x, T());
            float pp[G];
            lds_get<G>(pst, j * SPI + vsub, pp);
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
              for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(pp[g], x[e], acc[g][e]);
          }
          wave_lds_sync();  // and before the next tile overwrites it
        }
      }
    };
    constexpr int kStep = WAVES * UA;
    u32x4_t kr2[UA][kChunks], vr2[UA][kVLoads];
    // The new token's terms are computed once the first tile is done (their
    // inputs, requested before it, have arrived by then), or after the loop by
    // a wave with no tile.
    bool new_pending = true;
    for (int t0 = wave * UA; t0 < ntiles; t0 += 2 * kStep) {
      load_set(kr2, vr2, t0 + kStep);
      process(kr, vr, t0);
      if (new_pending) {
        phase_stamp<T>(P, tid, 1);
        new_token();
        new_pending = false;
      }
      load_set(kr, vr, t0 + 2 * kStep);
      process(kr2, vr2, t0 + kStep);
    }
    if (new_pending) new_token();
    phase_stamp<T>(P, tid, 2);

    // ---------------- Combine the waves ----------------
    // Each wave's (m_w, sum, acc) goes to LDS; after one barrier every thread
    // forms the workgroup's max and sum per query head and each wave's factor
    // exp2(m_w - M), in one fixed order (so every thread holds the same bits;
    // one workgroup per pair: the new token included with weight
    // exp2(s_new - M)). Head g's sum is the sum over row g of the wave (lanes
    // 16g .. 16g + 15).
    const float lrow = row_sum(lsum);
#pragma unroll
    for (int off = LPS; off < kWave; off <<= 1)
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] += __shfl_xor(acc[g][e], off, kWave);
    if (lane < LPS) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < EPL; ++e) sh_red[wave][g][vcol + e] = acc[g][e];
    }
    if (lane == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) sh_part[wave][g] = m_w[g];
    }
    if (r16 == 0 && grp < G) sh_part2[wave][grp] = lrow;
    __syncthreads();  // partials, raw logits and the new token visible
    float gm[G], gl[G], fw[WAVES][G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float M = SPLIT ? kNoMax : sh_snew[g];
#pragma unroll
      for (int w = 0; w < WAVES; ++w) M = fmaxf(M, sh_part[w][g]);
      float L = SPLIT ? 0.0f : __builtin_amdgcn_exp2f(sh_snew[g] - M);
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        fw[w][g] = __builtin_amdgcn_exp2f(sh_part[w][g] - M);
        L = fmaf(sh_part2[w][g], fw[w][g], L);
      }
      gm[g] = M;
      gl[g] = L;
    }
    if constexpr (!SPLIT) {
      settle_loads();  // only finished prologue loads and zero-fill tail loads are pending
#pragma unroll
      for (int j = 0; j < kOutPer; ++j) {
        const int idx = tid + j * NT;
        if (idx < G * D) {
          const int g = idx / D;
          const int d = idx - g * D;
          float o = 0.0f, fg[WAVES], mg = gm[0], lg = gl[0];
#pragma unroll
          for (int w = 0; w < WAVES; ++w) fg[w] = fw[w][0];
#pragma unroll
          for (int g2 = 1; g2 < G; ++g2) {
            if (g == g2) {
              mg = gm[g2];
              lg = gl[g2];
#pragma unroll
              for (int w = 0; w < WAVES; ++w) fg[w] = fw[w][g2];
            }
          }
#pragma unroll
          for (int w = 0; w < WAVES; ++w) o = fmaf(sh_red[w][g][d], fg[w], o);
          o = fmaf(__builtin_amdgcn_exp2f(sh_snew[g] - mg), to_f32(ov[j]), o);
          from_f32(o / lg, out_rows() + g * D + d);
        }
      }

      // ---------------- Score + argmin ----------------
      // score_i = ||v_i|| * sum_g exp2(s_{g,i} - M_g) / L_g from the raw logits
      // in LDS and the prefetched sidecar; (score, slot) argmin through DPP
      // and LDS, lowest slot on ties. With one victim per sequence every score
      // also goes to this pair's score vector for the sequence's deciding
      // workgroup.
      if (EVICT && scoring) {
        float inv_l[G];
#pragma unroll
        for (int g = 0; g < G; ++g) inv_l[g] = 1.0f / gl[g];
        const __amdgpu_buffer_rsrc_t rSc =
            make_rsrc(shared ? P.ws_score + static_cast<int64_t>(pair) * slots_pad : nullptr,
                      shared ? static_cast<uint32_t>(n) * 4u : 0u);
        auto score_batch = [&](int i0) {
#pragma unroll
          for (int k = 0; k < kScoreBatch; ++k) {
            const int i = i0 + k * NT;
            if (i < n && (!VAR || i != masked)) {
              float s[G];
              lds_get<G>(lds, i, s);
              float sc = __builtin_amdgcn_exp2f(s[0] - gm[0]) * inv_l[0];
#pragma unroll
              for (int g = 1; g < G; ++g) sc = fmaf(__builtin_amdgcn_exp2f(s[g] - gm[g]), inv_l[g], sc);
              sc = sc * vnb[k];
              if (shared) {
                const float one[1] = {sc};
                ws_store_g<1>(rSc, static_cast<uint32_t>(i) * 4u, one);
              }
              if (sc < best) {  // slots visited in increasing order: first minimum kept
                best = sc;
                best_i = i;
              }
            }
          }
        };
        // The first batch's sidecar was requested in the prologue; later
        // batches (budgets beyond NT * kScoreBatch slots) load their own.
        score_batch(P.sink + tid);
        for (int i0 = P.sink + tid + NT * kScoreBatch; i0 < n; i0 += NT * kScoreBatch) {
#pragma unroll
          for (int k = 0; k < kScoreBatch; ++k)
            vnb[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                rN, static_cast<int>((i0 + k * NT) * 4), 0, 0));
          score_batch(i0);
        }
        wave_argmin(best, best_i);
        if (lane == 0) {
          sh_best_score[wave] = best;
          sh_best_slot[wave] = best_i;
        }
        if (shared && tid == 0) ws_store(P.ws_nnorm + pair, sh_vn_new);
      }
    } else {
      // ---------------- Split: publish this split's partial state ----------------
      float* mine = P.ws_part + (wsr * wstride + split) * kPart;
      if (scoring) {
        // Raw logits of this split's slots for the last split's score.
        const __amdgpu_buffer_rsrc_t rW = make_rsrc(
            P.ws_logit + wsr * slots_pad * G, static_cast<uint32_t>(hi) * G * 4u);
        for (int i = tid; i < hi - lo; i += NT) {
          float x[G];
          lds_get<G>(lds, i, x);
          ws_store_g<G>(rW, static_cast<uint32_t>(lo + i) * G * 4u, x);
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        for (int d = tid; d < D; d += NT) {
          float o = 0.0f;
#pragma unroll
          for (int w = 0; w < WAVES; ++w) o = fmaf(sh_red[w][g][d], fw[w][g], o);
          ws_store(mine + 2 * G + g * D + d, o);
        }
      }
      if (tid == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          ws_store(mine + g, gm[g]);  // kNoMax for a split with no slots
          ws_store(mine + G + g, gl[g]);
        }
      }
      drain_stores();
      phase_stamp<T>(P, tid, 3);
      __syncthreads();
      if (tid == 0)
        sh_ticket = __hip_atomic_fetch_add(P.arrive + wsr, 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      phase_stamp<T>(P, tid, 4);
    }
  } else {
    // ======== Phased loop: K stream, softmax and score, then V stream ========
    // For long streams: each wave keeps one stream in flight at a time, and
    // the score is taken mid-stream while the first V rows are in flight.
    float* pbuf = lds;  // p overwrites the logits in place
    // K and V reads of the current chunk [c0, c0 + cn) go through descriptors
    // that end where the chunk ends (whole tiles for K): the loops below always
    // request the next register set, and requests past the chunk return zeros
    // without moving data (so the compiler's load counting stays exact and
    // both register sets stay in flight).
    int cn = min(P.chunk, hi - lo);
    int ntiles = (cn + 15) >> 4;
    __amdgpu_buffer_rsrc_t rK = make_rsrc(K, static_cast<uint32_t>((lo + cn + 15) >> 4) * kTileBytes);
    __amdgpu_buffer_rsrc_t rV = make_rsrc(V, static_cast<uint32_t>(lo + cn) * kRowBytes);

    // First K tiles go out before anything else.
    u32x4_t kr[UA][kChunks];
    {
      const uint32_t off0 = static_cast<uint32_t>(lo >> 4) * kTileBytes + k_lane_offset(lane);
#pragma unroll
      for (int u = 0; u < UA; ++u)
#pragma unroll
        for (int c = 0; c < kChunks; ++c)
          kr[u][c] = bload16<POLICY>(
              rK, off0 + static_cast<uint32_t>(wave * UA + u) * kTileBytes + 1024u * c);
    }

    // Query operand in the MFMA A layout: lane = row (query head row % G) +
    // 16 * (16-byte chunk group); the same byte offsets as the key loads.
    u32x4_t qa[kChunks];
#pragma unroll
    for (int c = 0; c < kChunks; ++c)
      qa[c] = load16(qg + (r16 % G) * D + (64 * c + 16 * grp) / kBytes);

    // Sidecar of the slots this thread scores (the first kScoreBatch of them),
    // requested now so the score phase finds it in registers.
    const int sc_lo = max(lo, P.sink);
    const __amdgpu_buffer_rsrc_t rN =
        make_rsrc(P.vnorm + static_cast<int64_t>(pair) * slots_pad, static_cast<uint32_t>(hi) * 4u);
    float vnb[kScoreBatch];
    if (!SPLIT && scoring) {
#pragma unroll
      for (int k = 0; k < kScoreBatch; ++k)
        vnb[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            rN, static_cast<int>((sc_lo + tid + k * NT) * 4), 0, 0));
    }

    // Running softmax state, identical in every thread. One workgroup per
    // pair: the new token opens it with weight exp2(s_new - s_new) = 1. Split:
    // the partial holds the split's own slots only (the new token is added
    // once, when the partials are combined).
    float m_run[G], l_run[G], w_run[G];
    float acc[G][EPL];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m_run[g] = -INFINITY;
      l_run[g] = SPLIT ? 0.0f : 1.0f;
      w_run[g] = SPLIT ? 0.0f : 1.0f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] = 0.0f;
    }

    for (int c0 = lo; c0 < hi; c0 += P.chunk) {
      cn = min(P.chunk, hi - c0);
      ntiles = (cn + 15) >> 4;

      // ---------------- Phase A: logits of the chunk ----------------
      float wmax[G];
#pragma unroll
      for (int g = 0; g < G; ++g) wmax[g] = -INFINITY;
      const uint32_t base_off = static_cast<uint32_t>(c0 >> 4) * kTileBytes + k_lane_offset(lane);
      if (c0 > lo) {  // first tiles of a later chunk (the first chunk's are already in flight)
        rK = make_rsrc(K, static_cast<uint32_t>((c0 + cn + 15) >> 4) * kTileBytes);
        rV = make_rsrc(V, static_cast<uint32_t>(c0 + cn) * kRowBytes);
#pragma unroll
        for (int u = 0; u < UA; ++u)
#pragma unroll
          for (int c = 0; c < kChunks; ++c)
            kr[u][c] = bload16<POLICY>(
                rK, base_off + static_cast<uint32_t>(wave * UA + u) * kTileBytes + 1024u * c);
      }
      // Two register sets of UA tiles: the next set is requested before the
      // current one is multiplied, so every wave keeps K loads in flight.
      auto qk_tiles = [&](const u32x4_t (&kt)[UA][kChunks], int t0) {
#pragma unroll
        for (int u = 0; u < UA; ++u) {
          if (t0 + u < ntiles) {
            f32x4_t s4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int c = 0; c < kChunks; ++c) s4 = mfma_chunk(qa[c], kt[u][c], s4, T());
            const int i = (t0 + u) * 16 + r16;
            float s[G];
            const bool live = i < cn && (!VAR || c0 + i != masked);
#pragma unroll
            for (int g = 0; g < G; ++g) {
              s[g] = live ? s4[g] * P.scale_log2 : -INFINITY;
              wmax[g] = fmaxf(wmax[g], s[g]);
            }
            if (grp == 0) lds_put<G>(lds, i, s);
          }
        }
      };
      auto load_tiles = [&](u32x4_t (&kt)[UA][kChunks], int t0) {
#pragma unroll
        for (int u = 0; u < UA; ++u)
#pragma unroll
          for (int c = 0; c < kChunks; ++c)
            kt[u][c] = bload16<POLICY>(
                rK, base_off + static_cast<uint32_t>(t0 + u) * kTileBytes + 1024u * c);
      };
      constexpr int kStepA = WAVES * UA;
      u32x4_t kr2[UA][kChunks];
      for (int t0 = wave * UA; t0 < ntiles; t0 += 2 * kStepA) {
        load_tiles(kr2, t0 + kStepA);
        qk_tiles(kr, t0);
        load_tiles(kr, t0 + 2 * kStepA);
        qk_tiles(kr2, t0 + kStepA);
      }

      phase_stamp<T>(P, tid, 1);
      // First V rows of the chunk go out before the softmax bookkeeping.
      const int nq = (cn + SPI - 1) / SPI;
      const uint32_t vbase = static_cast<uint32_t>(c0 + vsub) * kRowBytes + vcol * kBytes;
      constexpr int kStepB = WAVES * UB;
      u32x4_t vr[UB], vr2[UB];
#pragma unroll
      for (int u = 0; u < UB; ++u)
        vr[u] = bload16<POLICY>(rV, vbase + static_cast<uint32_t>((wave * UB + u) * SPI) * kRowBytes);
#pragma unroll
      for (int u = 0; u < UB; ++u)
        vr2[u] = bload16<POLICY>(
            rV, vbase + static_cast<uint32_t>((wave * UB + kStepB + u) * SPI) * kRowBytes);

#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float m = wave_max(wmax[g]);
        if (lane == 0) sh_part[wave][g] = m;
      }
      if (c0 == lo) new_token();
      __syncthreads();  // logits, wave maxima and (first chunk) the new token visible

      // ---------------- A2: running max, p = exp2(s - M), sums ----------------
      float fac[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float m_old = c0 == lo ? sh_snew[g] : m_run[g];
        float m = m_old;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) m = fmaxf(m, sh_part[w][g]);
        m_run[g] = m;
        fac[g] = exp2f(m_old - m);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] *= fac[g];
      }
      float lpart[G];
#pragma unroll
      for (int g = 0; g < G; ++g) lpart[g] = 0.0f;
      // Split with a full cache: this pair's raw-logit area (no records otherwise).
      const __amdgpu_buffer_rsrc_t rW =
          make_rsrc(SPLIT && scoring ? P.ws_logit + wsr * slots_pad * G : nullptr,
                    SPLIT && scoring ? static_cast<uint32_t>(slots_pad) * G * 4u : 0u);
      for (int i = tid; i < ntiles * 16; i += NT) {  // masked slots hold -inf -> p = 0
        float x[G];
        lds_get<G>(lds, i, x);
        if (SPLIT && scoring && i < cn)  // raw logits for the last split's score
          ws_store_g<G>(rW, static_cast<uint32_t>(c0 + i) * G * 4u, x);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          x[g] = __builtin_amdgcn_exp2f(x[g] - m_run[g]);  // v_exp_f32; -inf -> 0
          lpart[g] += x[g];
        }
        lds_put<G>(pbuf, i, x);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float sum = wave_sum(lpart[g]);
        if (lane == 0) sh_part2[wave][g] = sum;
      }
      __syncthreads();  // p and the partial sums visible
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) sum += sh_part2[w][g];
        l_run[g] = fmaf(l_run[g], fac[g], sum);
        w_run[g] *= fac[g];
      }

      // ---------------- Phase C: score + argmin ----------------
      // One workgroup per pair: runs while the first V rows are in flight.
      // Only an evicting cache scores, and then the whole buffer is one chunk,
      // so M and L are final here. With one victim per sequence the scores go
      // to LDS and are published after the V pass (a global store here would
      // slow the transition).
      if (!SPLIT && EVICT && scoring) {
        float inv_l[G];
#pragma unroll
        for (int g = 0; g < G; ++g) inv_l[g] = 1.0f / l_run[g];
        for (int i0 = P.sink + tid; i0 < n; i0 += NT * kScoreBatch) {
          if (i0 != P.sink + tid) {  // later batches (the first one was prefetched)
#pragma unroll
            for (int k = 0; k < kScoreBatch; ++k)
              vnb[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                  rN, static_cast<int>((i0 + k * NT) * 4), 0, 0));
          }
#pragma unroll
          for (int k = 0; k < kScoreBatch; ++k) {
            const int i = i0 + k * NT;
            if (i < n && (!VAR || i != masked)) {
              float p[G];
              lds_get<G>(lds, i, p);
              float sc = p[0] * inv_l[0];
#pragma unroll
              for (int g = 1; g < G; ++g) sc = fmaf(p[g], inv_l[g], sc);
              sc = sc * vnb[k];
              if (shared) lds[P.chunk * G + i] = sc;
              if (sc < best) {  // slots visited in increasing order: first minimum kept
                best = sc;
                best_i = i;
              }
            }
          }
        }
        wave_argmin(best, best_i);
        if (lane == 0) {
          sh_best_score[wave] = best;
          sh_best_slot[wave] = best_i;
        }
      }

      // ---------------- Phase B: o += p * v over the chunk ----------------
      // Two register sets of UB rows, as for K.
      auto pv_rows = [&](const u32x4_t (&vt)[UB], int q0) {
#pragma unroll
        for (int u = 0; u < UB; ++u) {
          if (q0 + u < nq) {  // rows past the chunk have p = 0 (and load as 0 past n)
            const int r = (q0 + u) * SPI + vsub;
            float x[EPL];
            unpack16(vt[u], x, T());
            float p[G];
            lds_get<G>(pbuf, r, p);
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
              for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(p[g], x[e], acc[g][e]);
          }
        }
      };
      auto load_rows = [&](u32x4_t (&vt)[UB], int q0) {
#pragma unroll
        for (int u = 0; u < UB; ++u)
          vt[u] = bload16<POLICY>(rV, vbase + static_cast<uint32_t>((q0 + u) * SPI) * kRowBytes);
      };
      for (int q0 = wave * UB; q0 < nq; q0 += 2 * kStepB) {
        pv_rows(vr, q0);
        load_rows(vr, q0 + 2 * kStepB);
        pv_rows(vr2, q0 + kStepB);
        load_rows(vr2, q0 + 3 * kStepB);
      }
      if (c0 + P.chunk < hi) __syncthreads();  // the next chunk overwrites the LDS logits
    }

    if (lo >= hi) new_token();  // no slot for this workgroup: nothing streamed
    phase_stamp<T>(P, tid, 2);

    // ---------------- Phase D: cross-wave output reduction ----------------
#pragma unroll
    for (int off = LPS; off < kWave; off <<= 1)
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] += __shfl_xor(acc[g][e], off, kWave);
    if (lane < LPS) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < EPL; ++e) sh_red[wave][g][vcol + e] = acc[g][e];
    }
    __syncthreads();

    if constexpr (!SPLIT) {
      settle_loads();  // only finished prologue loads and zero-fill tail loads are pending
#pragma unroll
      for (int j = 0; j < kOutPer; ++j) {
        const int idx = tid + j * NT;
        if (idx < G * D) {
          const int g = idx / D;
          const int d = idx - g * D;
          float o = 0.0f;
#pragma unroll
          for (int w = 0; w < WAVES; ++w) o += sh_red[w][g][d];
          o = fmaf(w_run[g], to_f32(ov[j]), o);
          from_f32(o / l_run[g], out_rows() + g * D + d);
        }
      }
      if (EVICT && scoring && shared) {
        // One victim per sequence: publish this head's score vector (in LDS
        // since the score phase) and its new token's norm for the sequence's
        // deciding workgroup. Whole 16-byte groups; entries the score phase
        // skipped (sinks, the replaced slot) are never read back.
        const float* lsc = lds + P.chunk * G;
        const __amdgpu_buffer_rsrc_t rSc = make_rsrc(
            P.ws_score + static_cast<int64_t>(pair) * slots_pad, static_cast<uint32_t>(slots_pad) * 4u);
        for (int q4 = tid; 4 * q4 < n; q4 += NT) {
          const u32x4_t v4 = *reinterpret_cast<const u32x4_t*>(lsc + 4 * q4);
          __builtin_amdgcn_raw_buffer_store_b128(v4, rSc, 16 * q4, 0, kDeviceScope);
        }
        if (tid == 0) ws_store(P.ws_nnorm + pair, sh_vn_new);
      }
    } else {
      // ---------------- Split: publish this split's partial state ----------------
      float* mine = P.ws_part + (wsr * wstride + split) * kPart;
      for (int idx = tid; idx < G * D; idx += NT) {
        const int g = idx / D;
        const int d = idx - g * D;
        float o = 0.0f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) o += sh_red[w][g][d];
        ws_store(mine + 2 * G + idx, o);
      }
      if (tid < G) {
        ws_store(mine + tid, m_run[tid]);  // -inf for a split with no slots
        ws_store(mine + G + tid, l_run[tid]);
      }
      drain_stores();
      phase_stamp<T>(P, tid, 3);
      __syncthreads();
      if (tid == 0)
        sh_ticket = __hip_atomic_fetch_add(P.arrive + wsr, 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      phase_stamp<T>(P, tid, 4);
    }
  }

  if constexpr (SPLIT) {
    if (sh_ticket != S - 1) return;  // not the last split of the pair

    // ---------------- Last split: combine, score ----------------
    // Everything the combine and the first score batch read is requested
    // before any of it is used, in the order it is needed: every split's
    // (m, l) for this thread's query head, its partial outputs, then raw
    // logits and norms. The tail costs one memory round trip, not four.
    const float* part = P.ws_part + wsr * wstride * kPart;
    float ml[kMaxSplits][2];
    {
      const int g = tid & (G - 1);
#pragma unroll
      for (int s2 = 0; s2 < kMaxSplits; ++s2) {
        ml[s2][0] = s2 < S ? ws_load(part + s2 * kPart + g) : 0.0f;
        ml[s2][1] = s2 < S ? ws_load(part + s2 * kPart + G + g) : 0.0f;
      }
    }
    float op[kOutPer][kMaxSplits];
#pragma unroll
    for (int j = 0; j < kOutPer; ++j) {
      const int idx = min(tid + j * NT, G * D - 1);  // threads past G*D store nothing
#pragma unroll
      for (int s2 = 0; s2 < kMaxSplits; ++s2)
        op[j][s2] = s2 < S ? ws_load(part + s2 * kPart + 2 * G + idx) : 0.0f;
    }
    const __amdgpu_buffer_rsrc_t rL = make_rsrc(
        P.ws_logit + wsr * slots_pad * G, static_cast<uint32_t>(n) * G * 4u);
    const __amdgpu_buffer_rsrc_t rNa =
        make_rsrc(P.vnorm + static_cast<int64_t>(pair) * slots_pad, static_cast<uint32_t>(n) * 4u);
    constexpr int kLastBatch = 8;  // slots per thread with loads in flight together
    float vb[kLastBatch];
    float lg[kLastBatch][G];
    auto load_batch = [&](int i0) {
#pragma unroll
      for (int k = 0; k < kLastBatch; ++k) {
        vb[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            rNa, static_cast<int>((i0 + k * NT) * 4), 0, 0));
        ws_load_g<G>(rL, static_cast<uint32_t>(i0 + k * NT) * G * 4u, lg[k]);
      }
    };
    if (scoring) load_batch(P.sink + tid);

    if (tid < G) {  // global max and sum, new token included, fixed order
      const int g = tid;
      float M = sh_snew[g];
#pragma unroll
      for (int s2 = 0; s2 < kMaxSplits; ++s2)
        if (s2 < S) M = fmaxf(M, ml[s2][0]);
      float L = __builtin_amdgcn_exp2f(sh_snew[g] - M);
#pragma unroll
      for (int s2 = 0; s2 < kMaxSplits; ++s2) {
        if (s2 < S) {
          const float f = __builtin_amdgcn_exp2f(ml[s2][0] - M);
          sh_fac[s2][g] = f;
          L = fmaf(ml[s2][1], f, L);
        }
      }
      sh_gm[g] = M;
      sh_gl[g] = L;
    }
    __syncthreads();
    phase_stamp<T>(P, tid, 5);
    // Output values now, stores after the score: stores count in the same
    // counter as loads, so a store issued before the score's last loads
    // would have to be acknowledged before the score could finish.
    float ofin[kOutPer];
#pragma unroll
    for (int j = 0; j < kOutPer; ++j) {
      const int g = min((tid + j * NT) / D, G - 1);
      float o = 0.0f;
#pragma unroll
      for (int s2 = 0; s2 < kMaxSplits; ++s2)
        if (s2 < S) o = fmaf(op[j][s2], sh_fac[s2][g], o);
      o = fmaf(__builtin_amdgcn_exp2f(sh_snew[g] - sh_gm[g]), to_f32(ov[j]), o);
      ofin[j] = o / sh_gl[g];
    }
    if (scoring) {
      // Score every slot from the published raw logits: the same operations
      // as one workgroup per pair, so equal tokens get bit-equal scores.
      float inv_l[G], pm[G];  // the pair's sums and maxima
#pragma unroll
      for (int g = 0; g < G; ++g) {
        inv_l[g] = 1.0f / sh_gl[g];
        pm[g] = sh_gm[g];
      }
      const __amdgpu_buffer_rsrc_t rSc =
          make_rsrc(shared ? P.ws_score + static_cast<int64_t>(pair) * slots_pad : nullptr,
                    shared ? static_cast<uint32_t>(n) * 4u : 0u);
      for (int i0 = P.sink + tid; i0 < n; i0 += NT * kLastBatch) {
        if (i0 != P.sink + tid) load_batch(i0);  // the first batch is in flight already
#pragma unroll
        for (int k = 0; k < kLastBatch; ++k) {
          const int i = i0 + k * NT;
          if (i < n && (!VAR || i != masked)) {
            float p[G];
#pragma unroll
            for (int g = 0; g < G; ++g) p[g] = __builtin_amdgcn_exp2f(lg[k][g] - pm[g]);
            float sc = p[0] * inv_l[0];
#pragma unroll
            for (int g = 1; g < G; ++g) sc = fmaf(p[g], inv_l[g], sc);
            sc = sc * vb[k];
            if (shared) {
              const float one[1] = {sc};
              ws_store_g<1>(rSc, static_cast<uint32_t>(i) * 4u, one);
            }
            if (sc < best) {
              best = sc;
              best_i = i;
            }
          }
        }
      }
      phase_stamp<T>(P, tid, 6);
      wave_argmin(best, best_i);
      if (lane == 0) {
        sh_best_score[wave] = best;
        sh_best_slot[wave] = best_i;
      }
    }
#pragma unroll
    for (int j = 0; j < kOutPer; ++j) {
      const int idx = tid + j * NT;  // = g * D + d
      if (idx < G * D) from_f32(ofin[j], out_rows() + idx);
    }
    if (shared && scoring && tid == 0) ws_store(P.ws_nnorm + pair, sh_vn_new);
    if (tid == 0) __hip_atomic_store(P.arrive + wsr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // ---------------- Choice of the victim ----------------
  // One victim per pair: the cross-wave argmin of this workgroup, lowest slot
  // on ties. One victim per sequence: every KV head has published its score
  // vector; the last of them to finish sums them in head order and takes the
  // argmin. choice = -1 when there is no candidate.
  int choice = -1;
  bool decider = !shared;
  u32x4_t pre = {0u, 0u, 0u, 0u};  // one victim per sequence: prefetched new-token data
  float pre_norm = 0.0f;
  if (scoring) {
    if (!shared) {
      __syncthreads();  // every wave's best visible
      uint32_t bh = __float_as_uint(sh_best_score[0]);
      uint32_t bl = static_cast<uint32_t>(sh_best_slot[0]);
#pragma unroll
      for (int w = 1; w < WAVES; ++w)
        key_min(bh, bl, __float_as_uint(sh_best_score[w]), static_cast<uint32_t>(sh_best_slot[w]));
      choice = static_cast<int>(bl);
    } else {
      drain_stores();
      __syncthreads();
      if (tid == 0)
        sh_ticket = __hip_atomic_fetch_add(P.seq_arrive + b, 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      decider = sh_ticket == P.num_kv_heads - 1;
      if (decider) {
        const int hk = P.num_kv_heads;
        // Prefetch what the write of every head needs (same-step order):
        // this thread's first 16-byte chunk of a new row and, for tid < hk,
        // head tid's published ||v_new||.
        if (!deferred) {
          if (tid < hk * 2 * kRowLoads) {
            const int hh = tid / (2 * kRowLoads);
            const int j = tid - hh * (2 * kRowLoads);
            const int64_t pr = static_cast<int64_t>(b) * hk + hh;
            pre = j < kRowLoads ? load16(static_cast<const T*>(P.k_new) + pr * D + j * EPL)
                                : load16(static_cast<const T*>(P.v_new) + pr * D + (j - kRowLoads) * EPL);
          }
          if (tid < hk) pre_norm = ws_load(P.ws_nnorm + static_cast<int64_t>(b) * hk + tid);
        }
        // Head h's scores of slots 4q..4q+3 are one 16-byte load; a thread
        // has up to 8 heads x kQuadBatch such loads in flight, then sums the
        // heads in order.
        const __amdgpu_buffer_rsrc_t rS = make_rsrc(
            P.ws_score + static_cast<int64_t>(b) * hk * slots_pad,
            static_cast<uint32_t>(hk) * static_cast<uint32_t>(slots_pad) * 4u);
        constexpr int kQuadBatch = 2;
        float sbest = INFINITY;
        int sbest_i = 0x7fffffff;
        for (int q0 = tid; 4 * q0 < n; q0 += NT * kQuadBatch) {
          float tot[kQuadBatch][4];
#pragma unroll
          for (int kb = 0; kb < kQuadBatch; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) tot[kb][r] = 0.0f;
          for (int h0 = 0; h0 < hk; h0 += 8) {
            u32x4_t x[8][kQuadBatch];
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
              for (int kb = 0; kb < kQuadBatch; ++kb)
                x[j][kb] = __builtin_amdgcn_raw_buffer_load_b128(
                    rS,
                    static_cast<int>((static_cast<uint32_t>(min(h0 + j, hk - 1)) * slots_pad +
                                      4u * static_cast<uint32_t>(q0 + kb * NT)) * 4u),
                    0, kDeviceScope);
#pragma unroll
            for (int j = 0; j < 8; ++j)
              if (h0 + j < hk)
#pragma unroll
                for (int kb = 0; kb < kQuadBatch; ++kb)
#pragma unroll
                  for (int r = 0; r < 4; ++r) tot[kb][r] += __uint_as_float(x[j][kb][r]);
          }
#pragma unroll
          for (int kb = 0; kb < kQuadBatch; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int i = 4 * (q0 + kb * NT) + r;
              if (i >= P.sink && i < n && i != masked && tot[kb][r] < sbest) {
                sbest = tot[kb][r];
                sbest_i = i;
              }
            }
        }
        wave_argmin(sbest, sbest_i);
        if (lane == 0) {
          sh_best_score[wave] = sbest;
          sh_best_slot[wave] = sbest_i;
        }
        __syncthreads();
        uint32_t bh = __float_as_uint(sh_best_score[0]);
        uint32_t bl = static_cast<uint32_t>(sh_best_slot[0]);
#pragma unroll
        for (int w = 1; w < WAVES; ++w)
          key_min(bh, bl, __float_as_uint(sh_best_score[w]), static_cast<uint32_t>(sh_best_slot[w]));
        choice = static_cast<int>(bl);
        // Heads past the first NT have their ||v_new|| read and stored here,
        // inside the decision, so every read of another workgroup's data
        // follows the ticket on every path through the code (the first NT
        // were prefetched above and are stored with the rows below).
        if (!deferred && choice >= 0 && choice < P.budget)
          for (int hh = tid + NT; hh < hk; hh += NT)
            P.vnorm[(static_cast<int64_t>(b) * hk + hh) * slots_pad + choice] =
                ws_load(P.ws_nnorm + static_cast<int64_t>(b) * hk + hh);
        if (tid == 0)
          __hip_atomic_store(P.seq_arrive + b, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    if (choice < 0 || choice >= P.budget) choice = -1;
  }

  // ---------------- In-place write of the new token ----------------
  int slot;
  if (!deferred) {
    if (!overwrite) {
      slot = n;
    } else if (!shared) {
      slot = choice;
    } else {
      // One victim per sequence: its deciding workgroup stores the new token
      // of every KV head of the sequence (each head's reads are done: it took
      // its ticket after them).
      if (!decider) return;
      const int hk = P.num_kv_heads;
      if (choice >= 0) {
        for (int idx = tid; idx < hk * 2 * kRowLoads; idx += NT) {
          const int hh = idx / (2 * kRowLoads);
          const int j = idx - hh * (2 * kRowLoads);
          const int64_t pr = static_cast<int64_t>(b) * hk + hh;
          if (j < kRowLoads) {
            char* Kh = reinterpret_cast<char*>(static_cast<T*>(P.kc_w) + pr * P.pair_elems);
            store16(Kh + k_chunk_offset<kRowBytes>(choice, j),
                    idx == tid ? pre : load16(static_cast<const T*>(P.k_new) + pr * D + j * EPL));
          } else {
            T* Vh = static_cast<T*>(P.vc_w) + pr * P.pair_elems + static_cast<int64_t>(choice) * D;
            store16(Vh + (j - kRowLoads) * EPL,
                    idx == tid ? pre
                               : load16(static_cast<const T*>(P.v_new) + pr * D + (j - kRowLoads) * EPL));
          }
        }
        // The first NT heads' ||v_new|| at the victim slot (prefetched).
        if (tid < hk)
          P.vnorm[(static_cast<int64_t>(b) * hk + tid) * slots_pad + choice] = pre_norm;
      }
      for (int hh = tid; hh < hk; hh += NT) P.evicted[static_cast<int64_t>(b) * hk + hh] = choice;
      return;
    }
  } else {
    slot = overwrite ? masked : n;
    if (scoring && decider) {
      if (!shared) {
        if (tid == 0) P.victim[pair] = choice;
      } else {
        for (int hh = tid; hh < P.num_kv_heads; hh += NT)
          P.victim[static_cast<int64_t>(b) * P.num_kv_heads + hh] = choice;
      }
    }
  }
  phase_stamp<T>(P, tid, 7);
  if (tid >= 2 * kRowLoads) return;
  if (slot >= P.budget) return;  // FULL cache already at capacity (the host prevents it)
  if (tid == 0) {
    P.evicted[pair] = overwrite ? slot : -1;
    if (!overwrite) P.fill[pair] = n + 1;
  }
  if (slot < 0) return;  // no candidate (only with non-finite scores): nothing stored
  char* Kw = reinterpret_cast<char*>(static_cast<T*>(P.kc_w) + pair * P.pair_elems);
  T* Vw = static_cast<T*>(P.vc_w) + pair * P.pair_elems + static_cast<int64_t>(slot) * D;
  if (tid < kRowLoads)
    store16(Kw + k_chunk_offset<kRowBytes>(slot, tid), wrow);
  else
    store16(Vw + (tid - kRowLoads) * EPL, wrow);
  if (tid == 0) P.vnorm[static_cast<int64_t>(pair) * slots_pad + slot] = sh_vn_new;
}

// One workgroup per unit: the hardware hands the units out as workgroups
// finish. Split launches: unit = split * pairs + pair, equal parts.
template <typename T, int D, int G, bool EVICT, int WAVES, int UA, int UB, int POLICY, bool SPLIT,
          bool VAR, bool ILV>
__global__ __launch_bounds__(WAVES * kWave, WAVES >= 8 ? 1 : 2) void decode_kernel(DecodeParams P) {
  const ClockRecord clock_rec{P.wg_clock && threadIdx.x == 0 ? P.wg_clock + 4 * static_cast<size_t>(blockIdx.x)
                                                             : nullptr,
                              P.wg_clock ? __builtin_amdgcn_s_memrealtime() : 0};
  Part seg{0, 0, 1, 0, 1, -1, -1};
  if constexpr (SPLIT) {
    const int pair = static_cast<int>(blockIdx.x % static_cast<uint32_t>(P.pairs));
    seg = Part{pair, static_cast<int>(blockIdx.x / static_cast<uint32_t>(P.pairs)), P.splits, pair,
               P.splits, -1, -1};
  }
  decode_unit<T, D, G, EVICT, WAVES, UA, UB, POLICY, SPLIT, VAR, ILV>(P, blockIdx.x, threadIdx.x, seg);
}

// Stream launch of the evicting main path (no variant): workgroup w first
// takes its sk_q tiles of the run of pairs [sk_first, sk_first + sk_pairs)
// (a pair cut between workgroups becomes a split pair, combined by the last
// of its parts to finish; a pair held whole by w runs as usual), then the
// whole pairs w, w + grid, ... below sk_first. With sk_pairs = 0 this is
// whole pairs in turn. Every workgroup then does the same share of the
// layer's tiles, where one workgroup per pair would leave a round of
// resident workgroups part-full. A barrier separates the units, and the
// thread index is made opaque to the compiler at the top of each unit, so
// the lane roles and addresses are recomputed per unit rather than held in
// registers across the loop.
template <typename T, int D, int G, int WAVES, int UA, int UB, int POLICY, bool ILV>
__global__ __launch_bounds__(WAVES * kWave, WAVES >= 8 ? 1 : 2) void decode_kernel_stream(DecodeParams P) {
  const ClockRecord clock_rec{P.wg_clock && threadIdx.x == 0 ? P.wg_clock + 4 * static_cast<size_t>(blockIdx.x)
                                                             : nullptr,
                              P.wg_clock ? __builtin_amdgcn_s_memrealtime() : 0};
  const int w = blockIdx.x;
  bool first = true;
  if (w < P.sk_wgs) {
    const int64_t tn = P.sk_tiles;
    const int64_t total = static_cast<int64_t>(P.sk_pairs) * tn;
    const int64_t end = min(static_cast<int64_t>(w) * P.sk_q + P.sk_q, total);
    for (int64_t t = static_cast<int64_t>(w) * P.sk_q; t < end;) {
      const int row = static_cast<int>(t / tn);
      const int64_t base = row * tn;
      const int fw = static_cast<int>(base / P.sk_q);              // the pair's first workgroup
      const int lw = static_cast<int>((base + tn - 1) / P.sk_q);   // and its last
      if (!first) __syncthreads();  // every wave is done with the previous unit's LDS
      first = false;
      int tid = threadIdx.x;
      asm volatile("" : "+v"(tid));
      if (fw == lw) {
        decode_unit<T, D, G, true, WAVES, UA, UB, POLICY, false, false, ILV>(
            P, P.sk_first + row, tid, Part{0, 0, 1, 0, 1, -1, -1});
      } else {
        const Part seg{P.sk_first + row, w - fw, lw - fw + 1, row, P.sk_stride,
                       static_cast<int>(t - base), static_cast<int>(min(end - base, tn))};
        decode_unit<T, D, G, true, WAVES, UA, UB, POLICY, true, false, ILV>(P, 0, tid, seg);
      }
      t = base + tn;
    }
  }
  for (int unit = w; unit < P.sk_first; unit += gridDim.x) {
    if (!first) __syncthreads();
    first = false;
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    decode_unit<T, D, G, true, WAVES, UA, UB, POLICY, false, false, ILV>(P, unit, tid,
                                                                      Part{0, 0, 1, 0, 1, -1, -1});
  }
}

template <typename T, int D, int G, bool EVICT, bool SPLIT, bool VAR, int WAVES, bool ILV,
          int UA = 1, int UB = 4, int POLICY = kStream>
hipError_t launch_decode_t(const Geometry& geo, const LayerPtrs& L, const SplitWork& W, int splits,
                           const GridPlan& plan, const void* q, const void* k_new, const void* v_new,
                           void* out, int32_t* evicted, hipStream_t stream) {
  DecodeParams P;
  P.q = q;
  P.k_new = k_new;
  P.v_new = v_new;
  P.out = out;
  P.evicted = evicted;
  P.kc = L.k;
  P.vc = L.v;
  P.kc_w = L.k;
  P.vc_w = L.v;
  P.vnorm = L.vnorm;
  P.fill = L.fill;
  P.victim = L.victim;
  P.pair_elems = geo.pair_elems;
  P.num_q_heads = geo.num_q_heads;
  P.num_kv_heads = geo.num_kv_heads;
  P.budget = geo.budget;
  P.sink = geo.sink_size;
  P.scale_log2 = geo.scale * kLog2e;
  P.deferred = geo.order == 1;
  P.shared = geo.scope == 1;
  P.norm_l2 = geo.norm == 1;
  P.ws_score = W.score;
  P.ws_nnorm = W.new_norm;
  P.seq_arrive = W.seq_arrive;
  const int pairs = geo.batch * geo.num_kv_heads;
  P.pairs = pairs;
  P.splits = SPLIT ? splits : 1;
  P.ws_part = W.part;
  P.ws_logit = W.logit;
  P.arrive = W.arrive;
  P.wg_clock = W.wg_clock;
  P.wg_phase = W.wg_phase;
  P.order = EVICT ? nullptr : L.order;
  P.sk_first = P.sk_pairs = P.sk_tiles = P.sk_q = P.sk_wgs = P.sk_stride = 0;
  const size_t lds = SPLIT ? decode_split_lds_bytes(geo, splits, ILV) : decode_lds_bytes(geo, ILV);
  if (lds == 0) return hipErrorInvalidValue;
  // Phased loop, one workgroup per pair with one victim per sequence: the
  // pair's scores follow the logits in LDS.
  const size_t score_lds = !ILV && !SPLIT ? decode_score_lds_bytes(geo) : 0;
  P.chunk = static_cast<int32_t>((lds - score_lds) / (sizeof(float) * G));
  const dim3 block(WAVES * kWave);
  auto prepare = [lds](const void* k) {
    return lds > 65536 ? hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(lds))
                       : hipSuccess;
  };
  if constexpr (EVICT && !SPLIT && !VAR) {
    if (plan.grid > 0) {
      P.sk_first = plan.sk_first;
      P.sk_pairs = plan.sk_pairs;
      P.sk_tiles = plan.sk_tiles;
      P.sk_q = plan.sk_q;
      P.sk_wgs = plan.sk_wgs;
      P.sk_stride = plan.sk_stride;
      auto kern_s = &decode_kernel_stream<T, D, G, WAVES, UA, UB, POLICY, ILV>;
      const hipError_t e = prepare(reinterpret_cast<const void*>(kern_s));
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(kern_s, dim3(plan.grid), block, lds, stream, P);
      return hipGetLastError();
    }
  }
  auto kern = &decode_kernel<T, D, G, EVICT, WAVES, UA, UB, POLICY, SPLIT, VAR, ILV>;
  const hipError_t e = prepare(reinterpret_cast<const void*>(kern));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(SPLIT ? pairs * splits : pairs), block, lds, stream, P);
  return hipGetLastError();
}

// Dispatch over dtype, head_dim, group width, mode, split and variants for
// one workgroup size and loop kind.
template <int WAVES, bool ILV>
hipError_t launch_decode_waves(const Geometry& g, const LayerPtrs& L, const SplitWork& W, int splits,
                               const GridPlan& plan, const void* q, const void* k_new,
                               const void* v_new, void* out, int32_t* evicted, hipStream_t stream) {
  const bool var = g.order != 0 || g.scope != 0;
#define LF_LAUNCH(T, D, G, EVICT, SPLIT, VAR) \
  launch_decode_t<T, D, G, EVICT, SPLIT, VAR, WAVES, ILV>(g, L, W, SPLIT ? splits : 1, plan, q, k_new, v_new, out, evicted, stream)
#define LF_CASE(T, D, G)                                                                      \
  if (g.head_dim == D && g.group == G) {                                                     \
    if (g.mode != 0)                                                                         \
      return splits > 1 ? LF_LAUNCH(T, D, G, false, true, false)                             \
                        : LF_LAUNCH(T, D, G, false, false, false);                           \
    if (var)                                                                                 \
      return splits > 1 ? LF_LAUNCH(T, D, G, true, true, true) : LF_LAUNCH(T, D, G, true, false, true); \
    return splits > 1 ? LF_LAUNCH(T, D, G, true, true, false) : LF_LAUNCH(T, D, G, true, false, false); \
  }
  if (g.dtype == 1) {
    LF_CASE(uint16_t, 128, 1)
    LF_CASE(uint16_t, 128, 2)
    LF_CASE(uint16_t, 128, 4)
    LF_CASE(uint16_t, 64, 1)
    LF_CASE(uint16_t, 64, 2)
    LF_CASE(uint16_t, 64, 4)
  } else {
    LF_CASE(float, 128, 1)
    LF_CASE(float, 128, 2)
    LF_CASE(float, 128, 4)
    LF_CASE(float, 64, 1)
    LF_CASE(float, 64, 2)
    LF_CASE(float, 64, 4)
  }
#undef LF_CASE
#undef LF_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace
}  // namespace lf
