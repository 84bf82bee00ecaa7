// ceilings.hip -- device micro-benchmarks that put the attention kernels' roofline fractions in context.
//
// Not part of the attention path: bench.py loads this library (libceilings.so) to report, next to the
// prefill's MFMA fraction and the decode's HBM fraction, what this very device reaches on
//   * a pure matrix-core loop: back-to-back v_mfma_f32_32x32x16_bf16 (or 16x16x32) with operands held in
//     registers, fed from a caller buffer (random N(0,1) bf16 or a constant -- the chip's clock depends on
//     the data);
//   * a streaming read: every byte of a buffer read once with 16-byte loads, four in flight per lane;
//   * the split-KV decode's read pattern: caches [B, L, H, 128] bf16, workgroup = (split, KV head, batch),
//     64 rows of 256 B per step for K and for V;
//   * the issue cost of direct HBM -> LDS loads (global_load_lds_dwordx4, written as the prefill writes it):
//     cycles a wave spends issuing n such loads back to back (no wait), with 1 or 8 waves of a workgroup
//     issuing at once -- the prefill issues 32 of them per key tile, 4 per wave.
// Plus the CU count and peak engine clock the runtime reports.
//
// C ABI: every function returns a hipError_t value as int (0 = success, hipErrorInvalidValue for
// arguments that do not fit the kernel), launches on the given stream and does not synchronise it.
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kMfmaThreads = 256;
constexpr int kReadThreads = 256;

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Each lane loads four A and four B operand registers once, then issues iters x 32 MFMAs cycling over four
// independent accumulators (a dependent MFMA is four issues later, so the chain never stalls the pipe).
__global__ __launch_bounds__(kMfmaThreads) void mfma_loop_kernel(const bf16x8* __restrict__ ops, int64_t n_ops,
                                                                 float* __restrict__ sink, int iters) {
    const int64_t gid = (int64_t)blockIdx.x * kMfmaThreads + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * kMfmaThreads;
    bf16x8 a[4], b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        a[j] = ops[(gid + j * stride) % n_ops];
        b[j] = ops[(gid + (j + 4) * stride) % n_ops];
    }
    f32x16 c[4] = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int s = 0; s < 32; ++s)
            c[s & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s & 3], b[(s >> 2) & 3], c[s & 3], 0, 0, 0);
    }
    float r = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) r += c[j][i];
    sink[gid] = r;
}

// The same FLOPs with v_mfma_f32_16x16x32_bf16 (half the FLOPs per instruction): iters x 64 MFMAs over
// eight accumulators, A and B changing at the same pace as in mfma_loop_kernel.
__global__ __launch_bounds__(kMfmaThreads) void mfma16_loop_kernel(const bf16x8* __restrict__ ops, int64_t n_ops,
                                                                   float* __restrict__ sink, int iters) {
    const int64_t gid = (int64_t)blockIdx.x * kMfmaThreads + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * kMfmaThreads;
    bf16x8 a[4], b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        a[j] = ops[(gid + j * stride) % n_ops];
        b[j] = ops[(gid + (j + 4) * stride) % n_ops];
    }
    f32x4 c[8] = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int s = 0; s < 64; ++s)
            c[s & 7] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s & 3], b[(s >> 3) & 3], c[s & 7], 0, 0, 0);
    }
    float r = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) r += c[j][i];
    sink[gid] = r;
}

// Workgroup w reads vectors [w*per_wg, min((w+1)*per_wg, n_vec)) of the buffer.
__global__ __launch_bounds__(kReadThreads) void read_stream_kernel(const uint4* __restrict__ p, int64_t n_vec,
                                                                   int64_t per_wg, float* __restrict__ sink) {
    const int64_t begin = (int64_t)blockIdx.x * per_wg;
    const int64_t end = begin + per_wg < n_vec ? begin + per_wg : n_vec;
    uint32_t acc = 0;
    for (int64_t i = begin + threadIdx.x; i < end; i += 4 * kReadThreads) {
        const uint4 x0 = p[i];
        const uint4 x1 = i + kReadThreads < end ? p[i + kReadThreads] : make_uint4(0, 0, 0, 0);
        const uint4 x2 = i + 2 * kReadThreads < end ? p[i + 2 * kReadThreads] : make_uint4(0, 0, 0, 0);
        const uint4 x3 = i + 3 * kReadThreads < end ? p[i + 3 * kReadThreads] : make_uint4(0, 0, 0, 0);
        acc ^= x0.x ^ x0.y ^ x0.z ^ x0.w ^ x1.x ^ x1.y ^ x1.z ^ x1.w;
        acc ^= x2.x ^ x2.y ^ x2.z ^ x2.w ^ x3.x ^ x3.y ^ x3.z ^ x3.w;
    }
    if (acc == 0x9e3779b9u) sink[threadIdx.x] = 1.0f;   // keeps the loads; practically never taken
}

// Decode pattern: rows of 256 B (head_dim 128 bf16), 16 lanes per row, 16 rows per pass, 4 passes = one
// 64-key step, K and V.  Workgroup (split, h, b) covers keys [split*len, (split+1)*len).
__global__ __launch_bounds__(kReadThreads) void read_decode_kernel(const uint4* __restrict__ k,
                                                                   const uint4* __restrict__ v, int64_t L, int H,
                                                                   int64_t len, float* __restrict__ sink) {
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int row = threadIdx.x >> 4, ch = threadIdx.x & 15;
    const int64_t k0 = (int64_t)split * len;
    uint32_t acc = 0;
    for (int64_t t = k0; t < k0 + len; t += 64) {
        uint4 x[4], y[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t off = (((int64_t)b * L + t + row + 16 * i) * H + h) * 16 + ch;
            x[i] = k[off];
            y[i] = v[off];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) acc ^= x[i].x ^ x[i].y ^ x[i].z ^ x[i].w ^ y[i].x ^ y[i].y ^ y[i].z ^ y[i].w;
    }
    if (acc == 0x9e3779b9u) sink[threadIdx.x] = 1.0f;
}

constexpr int kDmaThreads = 512;   // 8 waves, as the prefill workgroup
constexpr int kDmaMaxInst = 8;
constexpr int64_t kDmaBytesPerWg = 65536;   // each workgroup reads its own 64 KB; wave w from byte 8192*w

__device__ __forceinline__ void dma_load_16(const void* sbase, uint32_t voff, uint32_t lds_base) {
    uint32_t saved_m0;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved_m0)
        : "v"(voff), "s"(sbase), "s"(lds_base)
        : "memory");
}

// Waves < active issue n_inst direct loads of 1 KB each (lane l: 16 bytes at 1024*i + 16*l) into LDS slots
// ((8*wave + i) mod 64) KB, timed with s_memtime around the issue; then every wave waits for its loads.
// out[(wg*8 + wave)*2] = issue cycles, [+1] = issue + wait cycles (waves >= active: both about 0).
__global__ __launch_bounds__(kDmaThreads) void lds_dma_issue_kernel(const char* __restrict__ src, uint64_t* out,
                                                                    int n_inst, int active) {
    __shared__ __attribute__((aligned(1024))) char smem[65536];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const uint32_t lds = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)smem;
    const char* base = src + (int64_t)blockIdx.x * kDmaBytesPerWg + wave * 8192;
    __syncthreads();
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    if (wave < active)
        for (int i = 0; i < n_inst; ++i)
            dma_load_16(base, (uint32_t)(i * 1024 + lane * 16), lds + ((wave * 8 + i) & 63) * 1024);
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
    const uint64_t t2 = __builtin_amdgcn_s_memtime();
    __syncthreads();
    if (lane == 0) {
        out[((int64_t)blockIdx.x * 8 + wave) * 2] = t1 - t0;
        out[((int64_t)blockIdx.x * 8 + wave) * 2 + 1] = t2 - t0;
    }
}

// Four 1 KB direct loads per active wave issued as one block, timed as above.  FORM 1: M0 is set once and
// the loads step through LDS by their immediate offsets (0, 1024, 2048, 3072; the offset is added to the
// global address too, so every lane's per-load offset is the same 16*l).  FORM 2: M0 is set before every
// load, as with a separate base per load, and restored once after the four.  With check, each active wave
// then copies its 4 KB of LDS there (check[(wg*8 + wave)*4096 ..]), which shows where the loads landed.
template <int FORM>
__global__ __launch_bounds__(kDmaThreads) void lds_dma_issue4_kernel(const char* __restrict__ src, uint64_t* out,
                                                                     int active, uint4* check) {
    __shared__ __attribute__((aligned(1024))) char smem[65536];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const uint32_t lds = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)smem + wave * 4096;
    const char* base = src + (int64_t)blockIdx.x * kDmaBytesPerWg + wave * 8192;
    const uint32_t o = (uint32_t)lane * 16;
    __syncthreads();
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    if (wave < active) {
        uint32_t saved_m0;
        if constexpr (FORM == 1) {
            asm volatile(
                "s_mov_b32 %0, m0\n\t"
                "s_mov_b32 m0, %3\n\t"
                "s_nop 0\n\t"
                "global_load_lds_dwordx4 %1, %2\n\t"
                "global_load_lds_dwordx4 %1, %2 offset:1024\n\t"
                "global_load_lds_dwordx4 %1, %2 offset:2048\n\t"
                "global_load_lds_dwordx4 %1, %2 offset:3072\n\t"
                "s_mov_b32 m0, %0"
                : "=&s"(saved_m0)
                : "v"(o), "s"(base), "s"(lds)
                : "memory");
        } else {
            asm volatile(
                "s_mov_b32 %0, m0\n\t"
                "s_mov_b32 m0, %3\n\t"
                "s_nop 0\n\t"
                "global_load_lds_dwordx4 %1, %2\n\t"
                "s_mov_b32 m0, %4\n\t"
                "s_nop 0\n\t"
                "global_load_lds_dwordx4 %1, %2 offset:1024\n\t"
                "s_mov_b32 m0, %5\n\t"
                "s_nop 0\n\t"
                "global_load_lds_dwordx4 %1, %2 offset:2048\n\t"
                "s_mov_b32 m0, %6\n\t"
                "s_nop 0\n\t"
                "global_load_lds_dwordx4 %1, %2 offset:3072\n\t"
                "s_mov_b32 m0, %0"
                : "=&s"(saved_m0)
                : "v"(o), "s"(base), "s"(lds), "s"(lds), "s"(lds), "s"(lds)
                : "memory");
        }
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
    const uint64_t t2 = __builtin_amdgcn_s_memtime();
    __syncthreads();
    if (lane == 0) {
        out[((int64_t)blockIdx.x * 8 + wave) * 2] = t1 - t0;
        out[((int64_t)blockIdx.x * 8 + wave) * 2 + 1] = t2 - t0;
    }
    if (check && wave < active) {
        const uint4* l = reinterpret_cast<const uint4*>(smem + wave * 4096);
        uint4* c = check + ((int64_t)blockIdx.x * 8 + wave) * 256;
#pragma unroll
        for (int i = 0; i < 4; ++i) c[i * 64 + lane] = l[i * 64 + lane];
    }
}

// LDS read bandwidth: 8 waves (one workgroup per CU) read a 64 KB LDS buffer in a loop, iters x 8 reads
// per wave, conflict-free (each read instruction covers consecutive 16-byte or 8-byte lane addresses),
// the values folded into a register so that no read is dropped.  FORM 0: ds_read_b128 (1 KB per
// instruction); FORM 1: ds_read_b64_tr_b16, the transposing read of the prefill's V operand (512 B).
// out[(wg*8 + wave)*2] = s_memtime cycles of the loop, [+1] = bytes this wave read.
typedef short lds_i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) lds_i16x4_t lds_i16x4_p;
template <int FORM>
__global__ __launch_bounds__(512) void lds_read_kernel(uint64_t* out, uint32_t* sink, int iters) {
    __shared__ __attribute__((aligned(1024))) uint4 buf[4096];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    for (int i = threadIdx.x; i < 4096; i += 512) buf[i] = make_uint4(i, 3u * i, 5u * i, 7u * i);
    __syncthreads();
    uint32_t acc = 0;
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int blk = (it * 8 + j + wave * 5) & 63;   // a 1 KB block of the buffer
            if constexpr (FORM == 0) {
                const uint4 v = buf[blk * 64 + lane];
                acc ^= v.x ^ v.y ^ v.z ^ v.w;
            } else {
                const char* p = reinterpret_cast<const char*>(buf) + blk * 1024 + lane * 8;
                const lds_i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_p*)(p));
                acc ^= (uint32_t)(uint16_t)v[0] ^ ((uint32_t)(uint16_t)v[1] << 16) ^ (uint32_t)(uint16_t)v[2] ^
                       ((uint32_t)(uint16_t)v[3] << 16);
            }
        }
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    __syncthreads();
    if (lane == 0) {
        out[((int64_t)blockIdx.x * 8 + wave) * 2] = t1 - t0;
        out[((int64_t)blockIdx.x * 8 + wave) * 2 + 1] = (uint64_t)iters * 8 * (FORM == 0 ? 1024 : 512);
    }
    if (acc == 0x9e3779b9u) sink[threadIdx.x] = acc;
}

}  // namespace

extern "C" {

// CU count and peak engine clock (kHz) of the current device.
int ceil_device_info(int* compute_units, int* clock_khz) {
    if (!compute_units || !clock_khz) return (int)hipErrorInvalidValue;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(compute_units, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(clock_khz, hipDeviceAttributeClockRate, dev);
    return (int)e;
}

// FLOPs of one ceil_mfma_loop call (either shape): workgroups * 4 waves * iters * 32 * 32768.
double ceil_mfma_loop_flops(int32_t workgroups, int32_t iters) {
    return (double)workgroups * (kMfmaThreads / 64) * iters * 32.0 * 32768.0;
}

// ops: n_ops 16-byte vectors of 8 bf16 (device); sink: >= workgroups*256 floats (device).
// shape 0: v_mfma_f32_32x32x16_bf16, 1: v_mfma_f32_16x16x32_bf16.
int ceil_mfma_loop(const void* ops, int64_t n_ops, float* sink, int64_t sink_elems, int32_t workgroups,
                   int32_t iters, int32_t shape, void* stream) {
    if (!ops || !sink || n_ops < 1 || workgroups < 1 || iters < 1 || (reinterpret_cast<uintptr_t>(ops) & 15u) ||
        sink_elems < (int64_t)workgroups * kMfmaThreads || (shape != 0 && shape != 1))
        return (int)hipErrorInvalidValue;
    if (shape == 0)
        hipLaunchKernelGGL(mfma_loop_kernel, dim3(workgroups), dim3(kMfmaThreads), 0,
                           reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const bf16x8*>(ops), n_ops, sink,
                           iters);
    else
        hipLaunchKernelGGL(mfma16_loop_kernel, dim3(workgroups), dim3(kMfmaThreads), 0,
                           reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const bf16x8*>(ops), n_ops, sink,
                           iters);
    return (int)hipGetLastError();
}

// buf: bytes (a multiple of 16) of device memory, read once; sink: >= 256 floats.
int ceil_read_stream(const void* buf, int64_t bytes, float* sink, int64_t sink_elems, int32_t workgroups,
                     void* stream) {
    if (!buf || !sink || bytes < 16 || (bytes & 15) || (reinterpret_cast<uintptr_t>(buf) & 15u) || workgroups < 1 ||
        sink_elems < kReadThreads)
        return (int)hipErrorInvalidValue;
    const int64_t n_vec = bytes / 16;
    const int64_t per_wg = (n_vec + workgroups - 1) / workgroups;
    hipLaunchKernelGGL(read_stream_kernel, dim3(workgroups), dim3(kReadThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const uint4*>(buf), n_vec, per_wg,
                       sink);
    return (int)hipGetLastError();
}

// k, v: [batch, L, hkv, 128] bf16 caches (device); L must be a multiple of 64 * splits.
int ceil_read_decode(const void* k, const void* v, int64_t batch, int64_t L, int32_t hkv, int32_t splits,
                     float* sink, int64_t sink_elems, void* stream) {
    if (!k || !v || !sink || batch < 1 || batch > 65535 || hkv < 1 || hkv > 65535 || splits < 1 || L < 64 ||
        L % (64 * (int64_t)splits) != 0 || ((reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v)) & 15u) ||
        sink_elems < kReadThreads)
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(read_decode_kernel, dim3(splits, hkv, batch), dim3(kReadThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const uint4*>(k),
                       reinterpret_cast<const uint4*>(v), L, hkv, L / splits, sink);
    return (int)hipGetLastError();
}

// src: >= workgroups * 65536 bytes (device, 16-byte aligned); out: >= workgroups * 16 uint64 (device);
// 1 <= n_inst <= 8, 1 <= active_waves <= 8.
int ceil_lds_dma_issue(const void* src, int64_t src_bytes, uint64_t* out, int64_t out_elems, int32_t workgroups,
                       int32_t n_inst, int32_t active_waves, void* stream) {
    if (!src || !out || workgroups < 1 || n_inst < 1 || n_inst > kDmaMaxInst || active_waves < 1 ||
        active_waves > 8 || src_bytes < (int64_t)workgroups * kDmaBytesPerWg || out_elems < (int64_t)workgroups * 16 ||
        (reinterpret_cast<uintptr_t>(src) & 15u))
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(lds_dma_issue_kernel, dim3(workgroups), dim3(kDmaThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const char*>(src), out, n_inst,
                       active_waves);
    return (int)hipGetLastError();
}

// The four-load forms above (form 1 or 2); arguments as ceil_lds_dma_issue with n_inst = 4, plus check:
// null, or >= workgroups * 8 * 4096 bytes of device memory (16-byte aligned) for the LDS contents.
int ceil_lds_dma_issue4(const void* src, int64_t src_bytes, uint64_t* out, int64_t out_elems, int32_t workgroups,
                        int32_t form, int32_t active_waves, void* check, int64_t check_bytes, void* stream) {
    if (!src || !out || workgroups < 1 || (form != 1 && form != 2) || active_waves < 1 || active_waves > 8 ||
        src_bytes < (int64_t)workgroups * kDmaBytesPerWg || out_elems < (int64_t)workgroups * 16 ||
        (reinterpret_cast<uintptr_t>(src) & 15u) ||
        (check && (check_bytes < (int64_t)workgroups * 8 * 4096 || (reinterpret_cast<uintptr_t>(check) & 15u))))
        return (int)hipErrorInvalidValue;
    uint4* c = reinterpret_cast<uint4*>(check);
    if (form == 1)
        hipLaunchKernelGGL(lds_dma_issue4_kernel<1>, dim3(workgroups), dim3(kDmaThreads), 0,
                           reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const char*>(src), out, active_waves, c);
    else
        hipLaunchKernelGGL(lds_dma_issue4_kernel<2>, dim3(workgroups), dim3(kDmaThreads), 0,
                           reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const char*>(src), out, active_waves, c);
    return (int)hipGetLastError();
}

// LDS read bandwidth (form 0: ds_read_b128, 1: ds_read_b64_tr_b16).  out: >= workgroups * 16 uint64;
// sink: >= 512 uint32 (device; written only in the impossible case that keeps the reads alive).
int ceil_lds_read(uint64_t* out, int64_t out_elems, uint32_t* sink, int64_t sink_elems, int32_t workgroups,
                  int32_t form, int32_t iters, void* stream) {
    if (!out || !sink || workgroups < 1 || (form != 0 && form != 1) || iters < 1 ||
        out_elems < (int64_t)workgroups * 16 || sink_elems < 512)
        return (int)hipErrorInvalidValue;
    if (form == 0)
        hipLaunchKernelGGL(lds_read_kernel<0>, dim3(workgroups), dim3(512), 0, reinterpret_cast<hipStream_t>(stream),
                           out, sink, iters);
    else
        hipLaunchKernelGGL(lds_read_kernel<1>, dim3(workgroups), dim3(512), 0, reinterpret_cast<hipStream_t>(stream),
                           out, sink, iters);
    return (int)hipGetLastError();
}

}  // extern "C"
