// Machine-limit probes used by the benchmark to put the decode's rates next
// to what this chip reaches on plain work of each kind:
//   - a streaming read of a large buffer (the HBM ceiling a kernel that only
//     reads can reach), 16-byte loads, several in flight per lane;
//   - a loop of independent bf16 matrix instructions, 16x16x32, with no
//     memory traffic at all (the matrix-core ceiling), which also samples
//     the shader clock against the constant 100 MHz real-time counter;
//   - LDS reads of the two kinds the decode issues: 16-byte reads of key
//     fragments (rows 1152 bytes apart, XOR-swizzled chunks) and transposed
//     8-byte reads of value fragments, 8 waves per compute unit;
//   - matrix instructions in one wave of a SIMD beside plain vector work
//     (fused multiply-adds or exponentials) in the other, and each alone:
//     whether the two kinds of work share a SIMD's time or overlap;
//   - the page copies of the 64-row decode on their own: four waves copy
//     36 KiB slots HBM/L2 -> LDS by LDS-DMA into a four-slot ring, two slots
//     ahead, one barrier per slot, with the other four waves idle, reading
//     key fragments from LDS, or running matrix instructions beside them.

#include <hip/hip_runtime.h>
#include <stdint.h>

#pragma clang diagnostic ignored "-Winline-asm"

namespace mla {

typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 pbf16x8;
typedef __attribute__((ext_vector_type(4))) float pf32x4;
typedef __attribute__((ext_vector_type(4))) int i32x4p;

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;  // 16-byte loads in flight per lane

// Every lane reads kStreamUnroll 16-byte vectors per trip, the workgroups
// striding over the buffer; the XOR of everything read goes to one word per
// workgroup so that no load is dead.
__global__ void __launch_bounds__(kStreamThreads)
    probe_stream_read_kernel(const u32x4* __restrict__ src, size_t n_vec,
                             unsigned* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kStreamThreads * kStreamUnroll;
  u32x4 acc = {0u, 0u, 0u, 0u};
  size_t i = (size_t)blockIdx.x * kStreamThreads * kStreamUnroll + threadIdx.x;
  for (; i + (size_t)(kStreamUnroll - 1) * kStreamThreads < n_vec; i += stride) {
    u32x4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u)
      v[u] = __builtin_nontemporal_load(src + i + (size_t)u * kStreamThreads);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u];
  }
  // the ragged end: this lane's remaining positions of its last group (every
  // later group starts past the end, since stride > (kStreamUnroll - 1) * threads)
#pragma unroll
  for (int u = 0; u < kStreamUnroll - 1; ++u)
    if (i + (size_t)u * kStreamThreads < n_vec) acc ^= src[i + (size_t)u * kStreamThreads];
  __shared__ unsigned red[kStreamThreads];
  red[threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned x = 0;
    for (int t = 0; t < kStreamThreads; ++t) x ^= red[t];
    sink[blockIdx.x] = x;
  }
}

constexpr int kMfmaThreads = 512;  // 8 waves: two per SIMD
constexpr int kMfmaChains = 4;     // independent accumulators per wave

// iters x kMfmaChains matrix instructions per wave.  Block 0, thread 0 also
// records the shader-clock and real-time counters around its loop.
__global__ void __launch_bounds__(kMfmaThreads)
    probe_mfma_kernel(int iters, float* __restrict__ sink, unsigned long long* __restrict__ clk) {
  const int lane = threadIdx.x & 63;
  pbf16x8 a, b;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    a[k] = (__bf16)(0.001f * (float)(lane + k));
    b[k] = (__bf16)(0.002f * (float)(lane - k));
  }
  pf32x4 c[kMfmaChains];
#pragma unroll
  for (int k = 0; k < kMfmaChains; ++k) c[k] = pf32x4{0.f, 0.f, 0.f, 0.f};
  unsigned long long t0 = 0, r0 = 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    t0 = __builtin_readcyclecounter();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < kMfmaChains; ++k)
      c[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kMfmaChains; ++k) s += c[k][0] + c[k][1] + c[k][2] + c[k][3];
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    const unsigned long long t1 = __builtin_readcyclecounter();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    clk[0] = t1 - t0;
    clk[1] = r1 - r0;
  }
  sink[(size_t)blockIdx.x * kMfmaThreads + threadIdx.x] = s;
}

constexpr int kLdsProbeBytes = 65536;
constexpr int kLdsProbeThreads = 512;
typedef __attribute__((ext_vector_type(4))) short pi16x4;

// iters x 16 LDS reads per lane, of kind kTr (0: ds_read_b128 at the decode's
// key-fragment addresses, 1: ds_read_b64_tr_b16 at its value-fragment
// addresses), the pattern moved by 16 bytes per trip; every address is
// masked into the 64 KiB buffer.  Workgroup 0, thread 0 records the
// shader-clock cycles of its loop.
template <int kTr>
__global__ void __launch_bounds__(kLdsProbeThreads)
    probe_lds_kernel(int iters, int* __restrict__ sink, unsigned long long* __restrict__ clk) {
  __shared__ __attribute__((aligned(16))) char buf[kLdsProbeBytes];
  typedef __attribute__((address_space(3))) char lds_char;
  const int tid = threadIdx.x, lane = tid & 63;
  for (int i = tid; i < kLdsProbeBytes / 4; i += kLdsProbeThreads) ((int*)buf)[i] = i * 7 + 1;
  __syncthreads();
  const int l16 = lane & 15, g = lane >> 4;
  int off;
  if (kTr == 0) {
    const int sw = l16 & 7;
    off = l16 * 1152 + 16 * (g ^ (sw & 3)) + ((sw & 4) ? 64 : 0);
  } else {
    const int vt = 4 * g + (l16 >> 2);
    off = vt * 1152 + 16 * (((l16 & 3) >> 1) ^ (vt & 7)) + 8 * (l16 & 1);
  }
  off += (tid >> 6) * 128;
  constexpr int kMask = kTr == 0 ? kLdsProbeBytes - 16 : kLdsProbeBytes - 8;
  u32x4 acc = {0u, 0u, 0u, 0u};
  unsigned long long t0 = 0;
  if (blockIdx.x == 0 && tid == 0) t0 = __builtin_readcyclecounter();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int a = (off + k * 2304) & kMask;
      if (kTr == 0) {
        acc ^= *(const __attribute__((address_space(3))) u32x4*)((lds_char*)buf + a);
      } else {
        const pi16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) pi16x4*)((lds_char*)buf + a));
        acc.x ^= (unsigned)(unsigned short)v[0] | ((unsigned)(unsigned short)v[1] << 16);
        acc.y ^= (unsigned)(unsigned short)v[2] | ((unsigned)(unsigned short)v[3] << 16);
      }
    }
    off += 16;
  }
  if (blockIdx.x == 0 && tid == 0) clk[0] = __builtin_readcyclecounter() - t0;
  sink[(size_t)blockIdx.x * kLdsProbeThreads + tid] = (int)(acc.x ^ acc.y ^ acc.z ^ acc.w);
}

constexpr int kIssueThreads = 512;  // waves w and w + 4 share a SIMD

// kind 0: waves 0-3 run iters x 4 independent bf16 16x16x32 matrix
// instructions, waves 4-7 nothing; kind 1: waves 4-7 run iters x 16
// independent fused multiply-adds, waves 0-3 nothing; kind 2: waves 4-7 run
// iters x 4 independent exponentials (v_exp_f32); kind 3 = kinds 0 and 1
// together, kind 4 = kinds 0 and 2 together.  Workgroup 0 records the
// shader-clock cycles of the loops of wave 0 (clk[0]) and wave 4 (clk[1]).
template <int kKind>
__global__ void __launch_bounds__(kIssueThreads)
    probe_issue_kernel(int iters, float* __restrict__ sink, unsigned long long* __restrict__ clk) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr bool kMat = kKind == 0 || kKind == 3 || kKind == 4;
  constexpr bool kFma = kKind == 1 || kKind == 3;
  constexpr bool kExp = kKind == 2 || kKind == 4;
  pbf16x8 a, b;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    a[k] = (__bf16)(0.001f * (float)(lane + k));
    b[k] = (__bf16)(0.002f * (float)(lane - k));
  }
  pf32x4 c[kMfmaChains];
#pragma unroll
  for (int k = 0; k < kMfmaChains; ++k) c[k] = pf32x4{0.f, 0.f, 0.f, 0.f};
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = 0.5f + 0.001f * (float)(lane + i);
  unsigned long long t0 = 0;
  const bool stamp = blockIdx.x == 0 && (tid == 0 || tid == 256);
  if (stamp) t0 = __builtin_readcyclecounter();
  if (wave < 4) {
    if (kMat) {
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < kMfmaChains; ++k)
          c[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[k], 0, 0, 0);
      }
    }
  } else if (kFma) {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = __builtin_fmaf(x[i], 0.999f, 0.0001f);
    }
  } else if (kExp) {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = __builtin_amdgcn_exp2f(-x[i]);
    }
  }
  if (stamp) clk[tid == 0 ? 0 : 1] = __builtin_readcyclecounter() - t0;
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kMfmaChains; ++k) s += c[k][0] + c[k][1] + c[k][2] + c[k][3];
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i];
  sink[(size_t)blockIdx.x * kIssueThreads + tid] = s;
}

constexpr int kRingSlot = 36864;  // 32 tokens x 1152 bytes
constexpr int kRingThreads = 512;
constexpr int kRingCopies = 9;    // 1 KiB copies per copying wave and slot

// One wave-wide copy, 16 bytes per lane, of voff + soff of the resource to
// LDS address lds + 16 lane (M0 carries the LDS base; no compiled code in
// this kernel uses M0).
__device__ __forceinline__ void ring_copy16(__attribute__((address_space(3))) char* lds, int voff,
                                            i32x4p rsrc, int soff) {
  const int m0 = __builtin_amdgcn_readfirstlane((int)(size_t)lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(m0), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}

template <int kImm>
__device__ __forceinline__ void ring_wait() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kImm);
  asm volatile("" ::: "memory");
}

// Workgroup g copies slots s % slots of its own region src + g * slots *
// 36864, in the decode's order: copying wave c (waves 4..7) moves 8-token
// block c of a slot (nine 1 KiB LDS-DMA loads, chunk offsets XOR-swizzled
// by token as the decode lays them out) into ring buffer s & 3, two slots
// ahead, and waits for its copies of slot i before the barrier that opens
// step i.  kKind 0: waves 0..3 only meet the barriers; 1: they read the
// step's slot as the score waves do (36 16-byte key-fragment reads per lane);
// 2: they run 68 bf16 16x16x32 matrix instructions per step (a 64-row
// step's matrix work on one SIMD).  Wave 4 of each workgroup records its
// loop's shader-clock cycles (clk[2 g]) and the mean time from the end of a
// slot's issue to the end of the wait for it (clk[2 g + 1]).
template <int kKind>
__global__ void __launch_bounds__(kRingThreads, 1)
    probe_copy_ring_kernel(const char* __restrict__ src, int slots, int steps,
                           int* __restrict__ sink, unsigned long long* __restrict__ clk) {
  typedef __attribute__((address_space(3))) char lds_char;
  __shared__ __attribute__((aligned(1024))) char ring_[4 * kRingSlot];
  lds_char* ring = (lds_char*)ring_;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const char* base = src + (size_t)blockIdx.x * slots * kRingSlot;
  int acc = 0;
  if (wave >= 4) {
    const int c = wave - 4, blk = c * 9216;
    int coff[kRingCopies];
#pragma unroll
    for (int k = 0; k < kRingCopies; ++k) {
      const int pc = 64 * k + lane, t = pc / 72, ch = pc - t * 72;
      coff[k] = t * 1152 + 16 * (ch ^ (t & 7));
    }
    auto rsrc = [&](int s) __attribute__((always_inline)) {
      const unsigned long long a = (unsigned long long)(base + (size_t)(s % slots) * kRingSlot);
      return i32x4p{__builtin_amdgcn_readfirstlane((int)(unsigned)a),
                    __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xFFFF)), kRingSlot,
                    0x00020000};
    };
    const unsigned long long t0 = __builtin_readcyclecounter();
    unsigned long long issued[2] = {0, 0}, lat = 0;
    for (int s = 0; s < 2; ++s) {
      const i32x4p r = rsrc(s);
#pragma unroll
      for (int k = 0; k < kRingCopies; ++k)
        ring_copy16(ring + s * kRingSlot + blk + 1024 * k, coff[k], r, blk);
    }
    for (int i = 0; i < steps; ++i) {
      ring_wait<0x0F70 | 9>();  // this wave's copies of slot i landed
      const unsigned long long tl = __builtin_readcyclecounter();
      if (i >= 2) lat += tl - issued[i & 1];
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      const i32x4p r = rsrc(i + 2);
#pragma unroll
      for (int k = 0; k < kRingCopies; ++k)
        ring_copy16(ring + ((i + 2) & 3) * kRingSlot + blk + 1024 * k, coff[k], r, blk);
      issued[i & 1] = __builtin_readcyclecounter();
    }
    ring_wait<0x0F70>();  // nothing may still fly when the wave ends
    if (c == 0 && lane == 0) {
      clk[2 * blockIdx.x] = __builtin_readcyclecounter() - t0;
      clk[2 * blockIdx.x + 1] = steps > 2 ? lat / (unsigned long long)(steps - 2) : 0;
    }
  } else {
    pbf16x8 q;
#pragma unroll
    for (int k = 0; k < 8; ++k) q[k] = (__bf16)(0.001f * (float)(lane + k));
    const int l16 = lane & 15, g = lane >> 4, sw = l16 & 7;
    const int kl = l16 * 1152 + 16 * (g ^ (sw & 3));
    const int ke = kl + ((sw & 4) ? 64 : 0), ko = kl - ((sw & 4) ? 64 : 0);
    for (int i = 0; i < steps; ++i) {
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if constexpr (kKind == 1) {
        const lds_char* kb = ring + (i & 3) * kRingSlot;
        u32x4 x = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int ks = 0; ks < 18; ++ks) {
          x ^= *(const __attribute__((address_space(3))) u32x4*)(kb + ((ks & 1) ? ko : ke) + 64 * ks);
          x ^= *(const __attribute__((address_space(3))) u32x4*)(kb + ((ks & 1) ? ko : ke) + 64 * ks +
                                                               16 * 1152);
        }
        acc ^= (int)(x[0] ^ x[1] ^ x[2] ^ x[3]);
        __builtin_amdgcn_s_waitcnt(0xC07F);  // reads done before the next copies land
      } else if constexpr (kKind == 2) {
        pf32x4 cc[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) cc[k] = pf32x4{(float)k, 0.f, 0.f, (float)i};
#pragma unroll
        for (int r = 0; r < 17; ++r)
#pragma unroll
          for (int k = 0; k < 4; ++k) cc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q, q, cc[k], 0, 0, 0);
        acc += (int)(cc[0][0] + cc[1][1] + cc[2][2] + cc[3][3]);
      }
    }
  }
  sink[(size_t)blockIdx.x * kRingThreads + threadIdx.x] = acc;
}

}  // namespace mla

extern "C" hipError_t mla_launch_probe_copy_ring(int kind, const void* src, int slots, int steps,
                                                 int blocks, int* sink, unsigned long long* clk,
                                                 hipStream_t stream) {
  const dim3 grid(blocks), block(mla::kRingThreads);
  const char* s = (const char*)src;
  switch (kind) {
    case 0: hipLaunchKernelGGL(mla::probe_copy_ring_kernel<0>, grid, block, 0, stream, s, slots, steps, sink, clk); break;
    case 1: hipLaunchKernelGGL(mla::probe_copy_ring_kernel<1>, grid, block, 0, stream, s, slots, steps, sink, clk); break;
    default: hipLaunchKernelGGL(mla::probe_copy_ring_kernel<2>, grid, block, 0, stream, s, slots, steps, sink, clk); break;
  }
  return hipGetLastError();
}

extern "C" hipError_t mla_launch_probe_issue(int kind, int iters, int blocks, float* sink,
                                             unsigned long long* clk, hipStream_t stream) {
  const dim3 grid(blocks), block(mla::kIssueThreads);
  switch (kind) {
    case 0: hipLaunchKernelGGL(mla::probe_issue_kernel<0>, grid, block, 0, stream, iters, sink, clk); break;
    case 1: hipLaunchKernelGGL(mla::probe_issue_kernel<1>, grid, block, 0, stream, iters, sink, clk); break;
    case 2: hipLaunchKernelGGL(mla::probe_issue_kernel<2>, grid, block, 0, stream, iters, sink, clk); break;
    case 3: hipLaunchKernelGGL(mla::probe_issue_kernel<3>, grid, block, 0, stream, iters, sink, clk); break;
    default: hipLaunchKernelGGL(mla::probe_issue_kernel<4>, grid, block, 0, stream, iters, sink, clk); break;
  }
  return hipGetLastError();
}

extern "C" hipError_t mla_launch_probe_lds(int kind, int iters, int blocks, int* sink,
                                           unsigned long long* clk, hipStream_t stream) {
  if (kind == 0)
    hipLaunchKernelGGL(mla::probe_lds_kernel<0>, dim3(blocks), dim3(mla::kLdsProbeThreads), 0,
                       stream, iters, sink, clk);
  else
    hipLaunchKernelGGL(mla::probe_lds_kernel<1>, dim3(blocks), dim3(mla::kLdsProbeThreads), 0,
                       stream, iters, sink, clk);
  return hipGetLastError();
}

extern "C" hipError_t mla_launch_probe_stream_read(const void* src, size_t bytes, unsigned* sink,
                                                   int blocks, hipStream_t stream) {
  hipLaunchKernelGGL(mla::probe_stream_read_kernel, dim3(blocks), dim3(mla::kStreamThreads), 0,
                     stream, (const mla::u32x4*)src, bytes / 16, sink);
  return hipGetLastError();
}

extern "C" hipError_t mla_launch_probe_mfma(int iters, int blocks, float* sink,
                                            unsigned long long* clk, hipStream_t stream) {
  hipLaunchKernelGGL(mla::probe_mfma_kernel, dim3(blocks), dim3(mla::kMfmaThreads), 0, stream,
                     iters, sink, clk);
  return hipGetLastError();
}
