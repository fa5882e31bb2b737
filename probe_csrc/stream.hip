// Plain HBM streaming kernels for gfx950: read only, write only and copy, at a
// chosen per-workgroup footprint. Not part of the normalization path: they
// measure what the memory system gives a pure-read, pure-write and 50/50
// read/write stream on this part, the reference the row-norm kernels' fraction
// of peak is read against. Built into libmbn_stream.so (a library of its own).
//
// A workgroup of LANES lanes moves LANES * CHUNKS 16-byte chunks (lane t owns
// chunks j * LANES + t), with the same non-temporal 16-byte loads and stores
// as the row-norm kernels: every chunk of a workgroup is in flight before the
// first one is consumed.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int LANES, int CHUNKS>
__global__ void __launch_bounds__(LANES) stream_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst) {
  const size_t base = (size_t)blockIdx.x * LANES * CHUNKS;
  u32x4 v[CHUNKS];
#pragma unroll
  for (int j = 0; j < CHUNKS; ++j) v[j] = __builtin_nontemporal_load(src + base + (size_t)j * LANES + threadIdx.x);
#pragma unroll
  for (int j = 0; j < CHUNKS; ++j) __builtin_nontemporal_store(v[j], dst + base + (size_t)j * LANES + threadIdx.x);
}

// The xor of everything read is stored only when it equals `key` (never, for
// the caller's data in practice), so the loads cannot be dropped; `sink`
// receives at most LANES chunks per workgroup.
template <int LANES, int CHUNKS>
__global__ void __launch_bounds__(LANES) stream_read(const u32x4* __restrict__ src, u32x4* __restrict__ sink,
                                                     uint32_t key) {
  const size_t base = (size_t)blockIdx.x * LANES * CHUNKS;
  u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < CHUNKS; ++j) acc ^= __builtin_nontemporal_load(src + base + (size_t)j * LANES + threadIdx.x);
  if (acc.x == key && acc.y == key) sink[threadIdx.x] = acc;
}

template <int LANES, int CHUNKS>
__global__ void __launch_bounds__(LANES) stream_write(u32x4* __restrict__ dst, uint32_t value) {
  const size_t base = (size_t)blockIdx.x * LANES * CHUNKS;
  const u32x4 v = {value, value, value, value};
#pragma unroll
  for (int j = 0; j < CHUNKS; ++j) __builtin_nontemporal_store(v, dst + base + (size_t)j * LANES + threadIdx.x);
}

// Copy whose 16-byte stores carry a chosen cache policy: global_store_dwordx4
// with the nt / sc0 / sc1 bits of POL (0: nt, 1: nt sc1, 2: sc1, 3: sc0 sc1),
// 256 lanes and CHUNKS chunks per lane. The loads are the compiler's (so its
// waits cover the stores' data operands); the stores are inline assembly, each
// followed by two wait states: on gfx950 a VALU instruction may overwrite the
// data registers of a store wider than 8 bytes only two wait states after it
// (the compiler inserts them after its own stores, not after inline assembly).
template <int CHUNKS, int POL>
__global__ void __launch_bounds__(256) stream_copy_policy(const u32x4* __restrict__ src, u32x4* __restrict__ dst) {
  const size_t base = (size_t)blockIdx.x * 256 * CHUNKS;
  u32x4 v[CHUNKS];
#pragma unroll
  for (int j = 0; j < CHUNKS; ++j) v[j] = __builtin_nontemporal_load(src + base + (size_t)j * 256 + threadIdx.x);
#pragma unroll
  for (int j = 0; j < CHUNKS; ++j) {
    u32x4* p = dst + base + (size_t)j * 256 + threadIdx.x;
    if constexpr (POL == 0) {
      __asm__ __volatile__("global_store_dwordx4 %0, %1, off nt\n\ts_nop 1" ::"v"(p), "v"(v[j]) : "memory");
    } else if constexpr (POL == 1) {
      __asm__ __volatile__("global_store_dwordx4 %0, %1, off nt sc1\n\ts_nop 1" ::"v"(p), "v"(v[j]) : "memory");
    } else if constexpr (POL == 2) {
      __asm__ __volatile__("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" ::"v"(p), "v"(v[j]) : "memory");
    } else {
      __asm__ __volatile__("global_store_dwordx4 %0, %1, off sc0 sc1\n\ts_nop 1" ::"v"(p), "v"(v[j]) : "memory");
    }
  }
}

// The QK-norm + RoPE kernel's memory access pattern with no arithmetic: for
// each token row of `row` 16-byte chunks, the first `qk` chunks (the q and k
// heads) are read and written back in place (v untouched), one workgroup of
// 256 lanes per token, every load issued before the first store, loads and
// stores non-temporal as in the kernel. The xor with `key` (0 from the host)
// keeps the stores from being folded away.
__global__ void __launch_bounds__(256) stream_qk_pattern(u32x4* __restrict__ qkv, int row, int qk, uint32_t key) {
  u32x4* t = qkv + (size_t)blockIdx.x * row;
  constexpr int kMax = 4;  // up to 4 * 256 chunks (16 KiB) of q and k per token
  u32x4 v[kMax];
#pragma unroll
  for (int j = 0; j < kMax; ++j) {
    const int k = j * 256 + threadIdx.x;
    if (k < qk) v[j] = __builtin_nontemporal_load(t + k);
  }
#pragma unroll
  for (int j = 0; j < kMax; ++j) {
    const int k = j * 256 + threadIdx.x;
    if (k < qk) __builtin_nontemporal_store(v[j] ^ key, t + k);
  }
}

typedef void (*PolicyCopy)(const u32x4*, u32x4*);
const PolicyCopy kPolicyCopies[2][4] = {
    {&stream_copy_policy<1, 0>, &stream_copy_policy<1, 1>, &stream_copy_policy<1, 2>, &stream_copy_policy<1, 3>},
    {&stream_copy_policy<8, 0>, &stream_copy_policy<8, 1>, &stream_copy_policy<8, 2>, &stream_copy_policy<8, 3>},
};

struct Shape {
  int lanes, chunks;
  void (*copy)(const u32x4*, u32x4*);
  void (*read)(const u32x4*, u32x4*, uint32_t);
  void (*write)(u32x4*, uint32_t);
};

#define MBN_STREAM_SHAPE(L, C) \
  Shape { L, C, &stream_copy<L, C>, &stream_read<L, C>, &stream_write<L, C> }

// Footprints per workgroup: 4, 8, 16, 32 and 64 KiB.
const Shape kShapes[] = {
    MBN_STREAM_SHAPE(256, 1), MBN_STREAM_SHAPE(512, 1), MBN_STREAM_SHAPE(1024, 1), MBN_STREAM_SHAPE(256, 4),
    MBN_STREAM_SHAPE(256, 8), MBN_STREAM_SHAPE(1024, 2), MBN_STREAM_SHAPE(256, 16),
};

const Shape* find(int lanes, int chunks) {
  for (const Shape& s : kShapes)
    if (s.lanes == lanes && s.chunks == chunks) return &s;
  return nullptr;
}

// 0 = ok, 1 = invalid (bytes not whole workgroups, misaligned pointer, no
// such shape), 3 = launch failed.
int check(const void* p, size_t bytes, int lanes, int chunks, const Shape** s) {
  *s = find(lanes, chunks);
  if (!*s || !p || ((uintptr_t)p & 15) != 0) return 1;
  const size_t per_wg = (size_t)lanes * chunks * 16;
  if (bytes == 0 || bytes % per_wg != 0 || bytes / per_wg > 0x7fffffffull) return 1;
  return 0;
}

}  // namespace

extern "C" {

__attribute__((visibility("default"))) int mbn_stream_copy(const void* src, void* dst, size_t bytes, int lanes,
                                                           int chunks, void* stream) {
  const Shape* s;
  int rc = check(src, bytes, lanes, chunks, &s);
  if (rc == 0) rc = check(dst, bytes, lanes, chunks, &s);
  if (rc) return rc;
  const size_t grid = bytes / ((size_t)lanes * chunks * 16);
  hipLaunchKernelGGL(s->copy, dim3((unsigned)grid), dim3(lanes), 0, (hipStream_t)stream,
                     (const u32x4*)src, (u32x4*)dst);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

// mbn_stream_copy with the kernel's own start and end recorded in two
// caller-created events (hipExtLaunchKernel), as the library's timed entry
// points do, so the copy and the row norm are timed alike.
__attribute__((visibility("default"))) int mbn_stream_copy_timed(const void* src, void* dst, size_t bytes,
                                                                 int lanes, int chunks, void* stream,
                                                                 void* start, void* stop) {
  const Shape* s;
  int rc = check(src, bytes, lanes, chunks, &s);
  if (rc == 0) rc = check(dst, bytes, lanes, chunks, &s);
  if (rc == 0 && (!start || !stop)) rc = 1;
  if (rc) return rc;
  const size_t grid = bytes / ((size_t)lanes * chunks * 16);
  hipExtLaunchKernelGGL(s->copy, dim3((unsigned)grid), dim3(lanes), 0, (hipStream_t)stream,
                        (hipEvent_t)start, (hipEvent_t)stop, 0, (const u32x4*)src, (u32x4*)dst);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

// The store-policy copy (stream_copy_policy): chunks 1 or 8 per lane of 256
// lanes, policy 0-3 as listed there.
__attribute__((visibility("default"))) int mbn_stream_copy_policy(const void* src, void* dst, size_t bytes,
                                                                  int chunks, int policy, void* stream) {
  const Shape* s;
  int rc = check(src, bytes, 256, chunks, &s);
  if (rc == 0) rc = check(dst, bytes, 256, chunks, &s);
  if (rc || (chunks != 1 && chunks != 8) || policy < 0 || policy > 3) return rc ? rc : 1;
  const size_t grid = bytes / ((size_t)256 * chunks * 16);
  hipLaunchKernelGGL(kPolicyCopies[chunks == 8][policy], dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4*)src, (u32x4*)dst);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

// stream_qk_pattern over T token rows of `row` chunks, the first `qk` of them
// read and written back (qk <= 1024 <= row). 0 = ok, 1 = invalid, 3 = launch
// failed.
__attribute__((visibility("default"))) int mbn_stream_qk_pattern(void* qkv, int64_t T, int row, int qk,
                                                                 void* stream) {
  if (!qkv || ((uintptr_t)qkv & 15) != 0 || T <= 0 || T > 0x7fffffff || qk <= 0 || qk > 1024 || row < qk) return 1;
  hipLaunchKernelGGL(stream_qk_pattern, dim3((unsigned)T), dim3(256), 0, (hipStream_t)stream, (u32x4*)qkv, row, qk,
                     0u);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

// sink: device buffer of at least lanes * 16 bytes (written only in the
// improbable case described above).
__attribute__((visibility("default"))) int mbn_stream_read(const void* src, void* sink, size_t bytes, int lanes,
                                                           int chunks, void* stream) {
  const Shape* s;
  int rc = check(src, bytes, lanes, chunks, &s);
  if (rc) return rc;
  if (!sink || ((uintptr_t)sink & 15) != 0) return 1;
  const size_t grid = bytes / ((size_t)lanes * chunks * 16);
  hipLaunchKernelGGL(s->read, dim3((unsigned)grid), dim3(lanes), 0, (hipStream_t)stream, (const u32x4*)src,
                     (u32x4*)sink, 0x9e3779b9u);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

__attribute__((visibility("default"))) int mbn_stream_write(void* dst, size_t bytes, int lanes, int chunks,
                                                            uint32_t value, void* stream) {
  const Shape* s;
  const int rc = check(dst, bytes, lanes, chunks, &s);
  if (rc) return rc;
  const size_t grid = bytes / ((size_t)lanes * chunks * 16);
  hipLaunchKernelGGL(s->write, dim3((unsigned)grid), dim3(lanes), 0, (hipStream_t)stream, (u32x4*)dst, value);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // extern "C"
