// gfx950 (MI355X) kernels around the decode step: the initial fill, sequence
// recycling, LDS sizing, and the choice of workgroup size for a decode launch.
// The decode kernel itself is in lf_decode.h, instantiated by lf_decode_w4.hip,
// lf_decode_w8.hip (phased loop) and lf_decode_w4i.hip, lf_decode_w8i.hip
// (interleaved loop).
#include "lf_decode.h"

namespace lf {
namespace {

// ---------------------------------------------------------------------------
// Initial fill: one wave per (pair, slot < n); copies the row (K into its tile
// position) and writes its norm. Only the listed sequences are touched, and
// slots at or beyond n keep what they held: no step reads them before they
// are written (K tiles past n are masked, V reads stop at n).
// ---------------------------------------------------------------------------
struct FillParams {
  const void* k;
  const void* v;
  void* kc;
  void* vc;
  float* vnorm;
  int32_t* fill;
  int32_t* victim;
  int64_t pair_elems;
  int32_t slots_pad;
  int32_t num_kv_heads;
  int32_t n_max;
  int32_t norm_l2;
  int32_t seq[kFillSeqPerLaunch];  // sequences filled by this launch
  int32_t n[kFillSeqPerLaunch];    // their lengths (>= 0)
};

template <typename T, int D>
__global__ __launch_bounds__(256) void fill_kernel(FillParams P) {
  constexpr int kBytes = Elem<T>::kBytes;
  constexpr int kRowBytes = D * kBytes;
  constexpr int kRowChunks = kRowBytes / 16;  // 16-byte chunks per row (<= 32)
  constexpr int EPL = 16 / kBytes;
  const int lane = threadIdx.x & (kWave - 1);
  const int slot = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int local_pair = blockIdx.y;
  const int bl = local_pair / P.num_kv_heads;
  const int h = local_pair - bl * P.num_kv_heads;
  const int b = P.seq[bl];
  const int64_t pair = static_cast<int64_t>(b) * P.num_kv_heads + h;
  const int nb = P.n[bl];
  if (slot >= P.slots_pad) return;
  if (slot == 0 && lane == 0) {
    P.fill[pair] = nb;
    P.victim[pair] = -1;
  }
  if (slot >= nb) return;
  char* Kd = reinterpret_cast<char*>(static_cast<T*>(P.kc) + pair * P.pair_elems);
  T* Vd = static_cast<T*>(P.vc) + pair * P.pair_elems + static_cast<int64_t>(slot) * D;
  const int64_t src = ((static_cast<int64_t>(b) * P.n_max + slot) * P.num_kv_heads + h) * D;
  const T* ks = static_cast<const T*>(P.k) + src;
  const T* vs = static_cast<const T*>(P.v) + src;
  if (lane < kRowChunks) {
    store16(Kd + k_chunk_offset<kRowBytes>(slot, lane), load16(ks + lane * EPL));
    store16(Vd + lane * EPL, load16(vs + lane * EPL));
  }
  const float nrm = wave_norm<T, D>(vs, lane, P.norm_l2 != 0);
  if (lane == 0) P.vnorm[pair * P.slots_pad + slot] = nrm;
}

// ---------------------------------------------------------------------------
// Sequence recycling: the listed sequences' pairs, in every layer, drop to 0
// tokens with no pending victim. One workgroup per (sequence, layer).
// ---------------------------------------------------------------------------
struct ResetParams {
  int32_t* fill;         // [layers][batch][num_kv_heads]
  int32_t* victim;       // same layout
  int32_t batch;
  int32_t num_kv_heads;
  int32_t count;
  int32_t seqs[kFillSeqPerLaunch];
};

__global__ __launch_bounds__(64) void seq_reset_kernel(ResetParams P) {
  const int j = blockIdx.x;
  if (j >= P.count) return;
  const int b = P.seqs[j];
  if (b < 0 || b >= P.batch) return;
  const int64_t base = (static_cast<int64_t>(blockIdx.y) * P.batch + b) * P.num_kv_heads;
  for (int hh = threadIdx.x; hh < P.num_kv_heads; hh += blockDim.x) {
    P.fill[base + hh] = 0;
    P.victim[base + hh] = -1;
  }
}

// ---------------------------------------------------------------------------
// Launch order of a layer's sequences (FULL mode): the values travel in the
// kernel arguments, so the write is stream-ordered and capturable.
// ---------------------------------------------------------------------------
struct OrderParams {
  int32_t* order;
  int32_t first;
  int32_t count;
  int32_t seq[kOrderPerLaunch];
};

__global__ __launch_bounds__(256) void set_order_kernel(OrderParams P) {
  for (int i = threadIdx.x; i < P.count; i += blockDim.x) P.order[P.first + i] = P.seq[i];
}

template <typename T, int D>
hipError_t launch_fill_t(const Geometry& geo, const LayerPtrs& L, const void* k, const void* v,
                         const int32_t* seq_host, const int32_t* n_host, int32_t count,
                         int32_t n_max, hipStream_t stream) {
  FillParams P;
  P.k = k;
  P.v = v;
  P.kc = L.k;
  P.vc = L.v;
  P.vnorm = L.vnorm;
  P.fill = L.fill;
  P.victim = L.victim;
  P.pair_elems = geo.pair_elems;
  P.slots_pad = geo.slots_pad;
  P.norm_l2 = geo.norm == 1;
  P.num_kv_heads = geo.num_kv_heads;
  P.n_max = n_max;
  int32_t longest = 0;
  for (int i = 0; i < kFillSeqPerLaunch; ++i) {
    P.seq[i] = i < count ? seq_host[i] : 0;
    P.n[i] = i < count ? n_host[i] : 0;
    if (i < count && n_host[i] > longest) longest = n_host[i];
  }
  // slot 0's wave always runs: it writes the fill level and clears the victim
  dim3 grid(longest > 0 ? (longest + 3) / 4 : 1, count * geo.num_kv_heads);
  hipLaunchKernelGGL((fill_kernel<T, D>), grid, dim3(256), 0, stream, P);
  return hipGetLastError();
}

}  // namespace

size_t device_lds_limit() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
    return 0;
  return static_cast<size_t>(v);
}

size_t decode_static_lds_bytes(const Geometry& g, int waves) {
  // sh_red[waves][group][head_dim] and sh_pst[waves][16 * group] floats, plus
  // the small per-wave arrays
  return static_cast<size_t>(waves) * g.group * (g.head_dim + 16) * sizeof(float) + 1024;
}

namespace {
bool decode_built(const Geometry& g) {
  return (g.head_dim == 64 || g.head_dim == 128) && (g.group == 1 || g.group == 2 || g.group == 4) &&
         (g.dtype == 0 || g.dtype == 1);
}
}  // namespace

size_t decode_score_lds_bytes(const Geometry& g) {
  return g.mode == 0 && g.scope == 1 ? static_cast<size_t>(g.slots_pad) * sizeof(float) : 0;
}

// Dynamic LDS of one workgroup per pair.
//   Evicting: the raw logits of the whole pair (the score needs every
//   slot's); the phased loop with one victim per sequence also keeps the
//   pair's scores.
//   FULL: the phased loop keeps the logits of one 2048-slot chunk at a time;
//   the interleaved loop keeps none (a nominal 16 bytes).
// 0 when the combination is not built or does not fit.
size_t decode_lds_bytes(const Geometry& g, bool ilv) {
  if (!decode_built(g)) return 0;
  if (g.mode != 0) {
    if (ilv) return 16;
    const size_t slots = g.slots_pad < static_cast<int>(kFullChunkSlots) ? g.slots_pad : kFullChunkSlots;
    return slots * g.group * sizeof(float);
  }
  const size_t logits = static_cast<size_t>(g.slots_pad) * g.group * sizeof(float);
  const size_t total = logits + (ilv ? 0 : decode_score_lds_bytes(g));
  return total > kEvictLdsCap ? 0 : total;
}

size_t decode_split_lds_bytes(const Geometry& g, int splits, bool ilv) {
  if (decode_lds_bytes(g, ilv) == 0 || splits < 1) return 0;
  if (g.mode != 0) return decode_lds_bytes(g, ilv);  // FULL: as without splits
  const int tiles = g.slots_pad / 16;
  const int per = (tiles + splits - 1) / splits;
  return static_cast<size_t>(per) * 16 * g.group * sizeof(float);  // one split's logits
}

size_t split_part_floats(const Geometry& g) {
  return 2 * static_cast<size_t>(g.group) + static_cast<size_t>(g.group) * g.head_dim;
}

hipError_t launch_decode(const Geometry& g, const LayerPtrs& L, const SplitWork& W, int splits, int waves,
                         bool ilv, const GridPlan& plan, const void* q, const void* k_new,
                         const void* v_new, void* out, int32_t* evicted, hipStream_t stream) {
  if (waves == 8)
    return ilv ? launch_decode_w8i(g, L, W, splits, plan, q, k_new, v_new, out, evicted, stream)
               : launch_decode_w8(g, L, W, splits, plan, q, k_new, v_new, out, evicted, stream);
  if (waves == 4)
    return ilv ? launch_decode_w4i(g, L, W, splits, plan, q, k_new, v_new, out, evicted, stream)
               : launch_decode_w4(g, L, W, splits, plan, q, k_new, v_new, out, evicted, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_seq_reset(const Geometry& g, int32_t num_layers, int32_t* fill, int32_t* victim,
                            const int32_t* seqs_host, int32_t count, hipStream_t stream) {
  if (count <= 0 || count > kFillSeqPerLaunch || num_layers <= 0) return hipErrorInvalidValue;
  ResetParams P;
  P.fill = fill;
  P.victim = victim;
  P.batch = g.batch;
  P.num_kv_heads = g.num_kv_heads;
  P.count = count;
  for (int i = 0; i < kFillSeqPerLaunch; ++i) P.seqs[i] = i < count ? seqs_host[i] : -1;
  hipLaunchKernelGGL(seq_reset_kernel, dim3(count, num_layers), dim3(64), 0, stream, P);
  return hipGetLastError();
}

hipError_t launch_set_order(int32_t* order, const int32_t* seq_host, int32_t first, int32_t count,
                            hipStream_t stream) {
  if (count <= 0 || count > kOrderPerLaunch || first < 0) return hipErrorInvalidValue;
  OrderParams P;
  P.order = order;
  P.first = first;
  P.count = count;
  for (int i = 0; i < kOrderPerLaunch; ++i) P.seq[i] = i < count ? seq_host[i] : 0;
  hipLaunchKernelGGL(set_order_kernel, dim3(1), dim3(256), 0, stream, P);
  return hipGetLastError();
}

hipError_t launch_fill(const Geometry& g, const LayerPtrs& L, const void* k, const void* v,
                       const int32_t* seq_host, const int32_t* n_host, int32_t count,
                       int32_t n_max, hipStream_t stream) {
  if (count <= 0 || count > kFillSeqPerLaunch) return hipErrorInvalidValue;
  if (g.dtype == 1) {
    if (g.head_dim == 128)
      return launch_fill_t<uint16_t, 128>(g, L, k, v, seq_host, n_host, count, n_max, stream);
    if (g.head_dim == 64)
      return launch_fill_t<uint16_t, 64>(g, L, k, v, seq_host, n_host, count, n_max, stream);
  } else {
    if (g.head_dim == 128)
      return launch_fill_t<float, 128>(g, L, k, v, seq_host, n_host, count, n_max, stream);
    if (g.head_dim == 64)
      return launch_fill_t<float, 64>(g, L, k, v, seq_host, n_host, count, n_max, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace lf
