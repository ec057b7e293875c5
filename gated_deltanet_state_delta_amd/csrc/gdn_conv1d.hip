// gdn_conv1d.hip -- causal depthwise conv1d over a ragged batch with a
// slot-indexed conv-state pool.
//
// Contract: "gated_delta_conv1d_fwd" (parameters and example).  Sequence b
// covers rows [off[b], off[b+1]) of x; channel c's window is the slot's K-1
// saved inputs (oldest first) followed by the sequence's inputs, and
//   out[t, c] = sum_{j < K} w[c, j] * window[p + j]   (p = t - off[b]),
// so w[c, K-1] multiplies the current input.  With write_state the slot then
// holds the last K-1 window entries.
//
// Design (HBM-bound streaming):
//  * conv1d_out_kernel: one thread per (run of `run` consecutive rows, group
//    of VE = 16 bytes of channels); a wave covers 64 consecutive channel
//    groups of one run, so every row access is a contiguous 1 KiB.  The
//    thread keeps the K taps of its channels and the K-1 previous inputs as a
//    sliding window in registers.  It finds the sequence of its first row
//    (a guess from the mean length, checked, else a binary search over the
//    offsets) and refills the window whenever a sequence starts: the slot's
//    saved inputs of a channel group are K-1 contiguous 16-byte chunks, then
//    the rows already seen are shifted in.  Inside a sequence, U rows (16,
//    or 8 for kernel sizes above 4) are loaded together before any is used.  Work items are dealt to the
//    XCDs in contiguous ranges (see the kernel).  The run length is picked on the
//    host from the mean sequence length (one row per thread for decode-like
//    batches, 32 rows for prefill).  Rows inside a batch are streamed with
//    non-temporal loads and stores.
//  * State write-back: the new window of a sequence is what the sliding
//    window holds after its last row.  When the whole sequence lies in one
//    run, its thread is the only reader of the slot and writes the window
//    back itself.  Sequences that span runs are written by
//    conv1d_state_kernel, launched after the output kernel on the same
//    stream, so no output thread can still be reading a slot it rewrites.
#include "gdn_device.hpp"
#include "gdn_kernels.hpp"

namespace gdn {

struct Conv1dParams {
  const void* x;
  const void* w;
  void* state;
  const uint32_t* slot;
  const uint32_t* off;
  void* out;
  int64_t T, x_st, o_st, max_slots;
  int C, n_seqs, run, write_state;
};

template <typename E> struct Vec16 { static constexpr int N = 16 / sizeof(E); };

// Element v of 16 raw bytes holding VE io elements, widened to fp32.
template <typename E> __device__ __forceinline__ float elem16(const u32x4& r, int v);
template <> __device__ __forceinline__ float elem16<float>(const u32x4& r, int v) {
  return __uint_as_float(r[v]);
}
template <> __device__ __forceinline__ float elem16<__bf16>(const u32x4& r, int v) {
  const uint32_t w = r[v >> 1];
  return __uint_as_float((v & 1) ? (w & 0xffff0000u) : (w << 16));
}

// VE fp32 values -> 16 raw bytes of io elements (bf16: round to nearest even).
template <typename E> __device__ __forceinline__ u32x4 pack16(const float* a);
template <> __device__ __forceinline__ u32x4 pack16<float>(const float* a) {
  return u32x4{__float_as_uint(a[0]), __float_as_uint(a[1]), __float_as_uint(a[2]), __float_as_uint(a[3])};
}
template <> __device__ __forceinline__ u32x4 pack16<__bf16>(const float* a) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = (uint32_t)__builtin_bit_cast(unsigned short, (__bf16)a[2 * i]) |
           ((uint32_t)__builtin_bit_cast(unsigned short, (__bf16)a[2 * i + 1]) << 16);
  return r;
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16_nt(void* p, const u32x4& v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// Bounds of sequence b: offsets clamped to [0, T]; a decreasing pair is empty.
__device__ __forceinline__ void seq_bounds(const Conv1dParams& p, int b, int64_t& s0, int64_t& s1) {
  s0 = min((int64_t)p.off[b], p.T);
  s1 = min((int64_t)p.off[b + 1], p.T);
  if (s1 < s0) s1 = s0;
}

// The sliding window of one channel group: win[i][v] is the input i rows
// back from the oldest (i = 0 oldest, H-1 newest) for channel c0 + v.
template <typename E, int K>
struct Window {
  static constexpr int VE = Vec16<E>::N, H = K - 1;
  float v[H > 0 ? H : 1][VE];

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < H; ++i)
#pragma unroll
      for (int e = 0; e < VE; ++e) v[i][e] = 0.f;
  }
  // The slot's saved inputs of channels c0 .. c0+VE-1: VE*H contiguous
  // elements (channel-major), i.e. H 16-byte chunks.
  __device__ __forceinline__ void load_saved(const E* slot_base) {
    u32x4 ch[H > 0 ? H : 1];
#pragma unroll
    for (int i = 0; i < H; ++i) ch[i] = ld16(slot_base + i * VE);
#pragma unroll
    for (int e = 0; e < VE; ++e)
#pragma unroll
      for (int i = 0; i < H; ++i) v[i][e] = elem16<E>(ch[(e * H + i) / VE], (e * H + i) % VE);
  }
  __device__ __forceinline__ void store_saved(E* slot_base) const {
    float flat[H > 0 ? H * VE : 1];
#pragma unroll
    for (int e = 0; e < VE; ++e)
#pragma unroll
      for (int i = 0; i < H; ++i) flat[e * H + i] = v[i][e];
#pragma unroll
    for (int i = 0; i < H; ++i) st16(slot_base + i * VE, pack16<E>(flat + i * VE));
  }
  __device__ __forceinline__ void shift_in(const float (&cur)[VE]) {
#pragma unroll
    for (int e = 0; e < VE; ++e) {
#pragma unroll
      for (int i = 0; i + 1 < H; ++i) v[i][e] = v[i + 1][e];
      if constexpr (H > 0) v[H - 1][e] = cur[e];
    }
  }
  __device__ __forceinline__ void shift_in_raw(const u32x4& raw) {
    float cur[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) cur[e] = elem16<E>(raw, e);
    shift_in(cur);
  }
  // Window before row t of a sequence starting at s0: the saved inputs (or
  // zeros) when t - s0 < H, then rows max(s0, t - H) .. t-1 shifted in.
  __device__ __forceinline__ void fill(const E* x, int64_t x_st, int c0, const E* slot_base, int64_t s0,
                                       int64_t t) {
    if constexpr (H > 0) {
      if (t - s0 < H) {
        if (slot_base) load_saved(slot_base);
        else zero();
      }
      for (int64_t r = max(s0, t - H); r < t; ++r) shift_in_raw(ld16(x + r * x_st + c0));
    }
  }
};

// One output row of VE channels from the current input and the window; the
// window then slides by one.
template <typename E, int K>
__device__ __forceinline__ u32x4 conv_step(const float (&w)[K][Vec16<E>::N], Window<E, K>& win,
                                           const u32x4& raw) {
  constexpr int VE = Vec16<E>::N, H = K - 1;
  float cur[VE], acc[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) {
    cur[e] = elem16<E>(raw, e);
    float a = w[H][e] * cur[e];
#pragma unroll
    for (int j = 0; j < H; ++j) a += w[j][e] * win.v[j][e];
    acc[e] = a;
  }
  win.shift_in(cur);
  return pack16<E>(acc);
}

// The sequence holding row t0: the mean-length guess if it holds, else the
// last sequence whose clamped start is <= t0 (binary search; offsets are
// non-decreasing).
__device__ __forceinline__ int find_seq(const Conv1dParams& p, int64_t t0) {
  const int n = p.n_seqs;
  int g = (int)min((int64_t)(n - 1), t0 * n / max(p.T, (int64_t)1));
  const int64_t a = min((int64_t)p.off[g], p.T), b = min((int64_t)p.off[g + 1], p.T);
  if (a <= t0 && t0 < b) return g;
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (min((int64_t)p.off[mid], p.T) <= t0) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

template <typename E, int K, int U>
__global__ void __launch_bounds__(256)
conv1d_out_kernel(const Conv1dParams p) {
  constexpr int VE = Vec16<E>::N, H = K - 1;
  const int ngroups = p.C / VE;
  // Workgroups are dealt to the 8 XCDs round robin; give each XCD a
  // contiguous range of work items instead, so the rows a run re-reads from
  // the run before it (same channels, 4 workgroups earlier for 8192
  // channels) sit in that XCD's own L2.
  const int nb = gridDim.x, xcd = blockIdx.x % 8, k = blockIdx.x / 8;
  const int lb = xcd * (nb / 8) + min(xcd, nb % 8) + k;
  const int64_t gid = (int64_t)lb * 256 + threadIdx.x;
  const int cg = (int)(gid % ngroups);
  const int64_t t0 = (gid / ngroups) * p.run;
  if (t0 >= p.T) return;
  const int c0 = cg * VE;
  const E* __restrict__ x = (const E*)p.x;
  E* __restrict__ out = (E*)p.out;

  float w[K][VE];
  {
    const E* wp = (const E*)p.w + (int64_t)c0 * K;
#pragma unroll
    for (int e = 0; e < VE; ++e)
#pragma unroll
      for (int j = 0; j < K; ++j) w[j][e] = to_f32(wp[e * K + j]);
  }

  int b = find_seq(p, t0);
  int64_t s0, s1;
  seq_bounds(p, b, s0, s1);
  E* slot_base = nullptr;  // this sequence's saved inputs, NULL outside the pool

  Window<E, K> win;
  bool filled = false;
  const int64_t tend = min(t0 + p.run, p.T);
  int64_t t = t0;
  while (t < tend) {
    if (t >= s1) {
      if (b + 1 >= p.n_seqs) break;  // rows after the last sequence
      ++b;
      seq_bounds(p, b, s0, s1);
      filled = false;
      continue;
    }
    if (t < s0) {  // rows no sequence covers
      t = s0;
      continue;
    }
    if (!filled) {
      const uint32_t sl = p.slot[b];
      slot_base = ((int64_t)sl < p.max_slots && H > 0) ? (E*)p.state + ((int64_t)sl * p.C + c0) * H : nullptr;
      win.fill(x, p.x_st, c0, slot_base, s0, t);
      filled = true;
    }
    const int64_t lim = min(tend, s1);
    if (t + U <= lim) {
      // U rows inside one sequence: all loads in flight together.  Rows are
      // streamed once (the few a later run re-reads for its window come back
      // from L2 or HBM): non-temporal loads and stores, 124 -> 105 us on
      // B4 x S4096 x 8192 channels.
      u32x4 raw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) raw[u] = ld16_nt(x + (t + u) * p.x_st + c0);
#pragma unroll
      for (int u = 0; u < U; ++u) st16_nt(out + (t + u) * p.o_st + c0, conv_step<E, K>(w, win, raw[u]));
      t += U;
    } else {
      st16(out + t * p.o_st + c0, conv_step<E, K>(w, win, ld16(x + t * p.x_st + c0)));
      t += 1;
    }
    // a sequence that lies wholly in this run has no other reader of its
    // slot: write the new window back now
    if constexpr (H > 0)
      if (t == s1 && p.write_state && slot_base && s0 >= t0) win.store_saved(slot_base);
  }
}

// New windows of the sequences that span runs, one thread per (sequence,
// channel group): the last K-1 entries of (saved ++ sequence).
template <typename E, int K>
__global__ void __launch_bounds__(256)
conv1d_state_kernel(const Conv1dParams p) {
  constexpr int VE = Vec16<E>::N, H = K - 1;
  const int ngroups = p.C / VE;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (int64_t)p.n_seqs * ngroups) return;
  const int b = (int)(gid / ngroups), c0 = (int)(gid % ngroups) * VE;
  const uint32_t sl = p.slot[b];
  if ((int64_t)sl >= p.max_slots) return;
  int64_t s0, s1;
  seq_bounds(p, b, s0, s1);
  // empty: the window is unchanged; one run: written by the output kernel
  if (s1 == s0 || s0 / p.run == (s1 - 1) / p.run) return;
  E* slot_base = (E*)p.state + ((int64_t)sl * p.C + c0) * H;
  Window<E, K> win;
  win.fill((const E*)p.x, p.x_st, c0, slot_base, s0, s1);
  win.store_saved(slot_base);
}

// Rows per thread of the output kernel, from the mean sequence length: one
// row for decode-like batches (one sequence per thread), 32 rows (two
// batches of 16) for long sequences; the window refill then re-reads K-1
// rows per 32.  Measured on B4 x S4096 x 8192 channels with non-temporal
// accesses: 16 rows 114 us, 32 rows 105 us, 64 rows 104 us, 128 rows 108 us.
static int conv1d_run(int64_t T, int n_seqs) {
  const int64_t mean = T / (n_seqs > 0 ? n_seqs : 1);
  int run = 1;
  while (run < 32 && 2 * run <= mean) run *= 2;
  return run;
}

template <typename E, int K>
static hipError_t launch_conv1d_k(const Conv1dParams& p, hipStream_t s) {
  constexpr int U = K <= 4 ? 16 : 8;  // rows loaded together (registers: U*4 + VE*(2K-1))
  const int64_t runs = (p.T + p.run - 1) / p.run;
  const int64_t threads = runs * (p.C / Vec16<E>::N);
  hipLaunchKernelGGL((conv1d_out_kernel<E, K, U>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, p);
  if (p.write_state && K > 1) {
    const int64_t n = (int64_t)p.n_seqs * (p.C / Vec16<E>::N);
    hipLaunchKernelGGL((conv1d_state_kernel<E, K>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

template <typename E>
static hipError_t dispatch_conv1d(const Conv1dParams& p, int K, hipStream_t s) {
  switch (K) {
    case 1: return launch_conv1d_k<E, 1>(p, s);
    case 2: return launch_conv1d_k<E, 2>(p, s);
    case 3: return launch_conv1d_k<E, 3>(p, s);
    case 4: return launch_conv1d_k<E, 4>(p, s);
    case 5: return launch_conv1d_k<E, 5>(p, s);
    case 6: return launch_conv1d_k<E, 6>(p, s);
    case 7: return launch_conv1d_k<E, 7>(p, s);
    case 8: return launch_conv1d_k<E, 8>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_conv1d(const gdn_conv1d_args& a, hipStream_t stream) {
  if (a.n_seqs == 0 || a.total_tokens == 0) return hipSuccess;
  Conv1dParams p;
  p.x = a.x; p.w = a.weight; p.state = a.conv_state; p.slot = a.slot_idx; p.off = a.row_offsets;
  p.out = a.out; p.T = a.total_tokens; p.x_st = a.x_stride_token; p.o_st = a.out_stride_token;
  p.max_slots = a.max_slots; p.C = a.conv_dim; p.n_seqs = a.n_seqs;
  p.run = conv1d_run(a.total_tokens, a.n_seqs);
  p.write_state = a.write_state != 0;
  if (a.io_dtype == GDN_BF16) return dispatch_conv1d<__bf16>(p, a.kernel_size, stream);
  return dispatch_conv1d<float>(p, a.kernel_size, stream);
}

}  // namespace gdn
