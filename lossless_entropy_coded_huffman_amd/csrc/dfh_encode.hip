// dfh_encode.hip -- device-side encoder for gfx950 (MI355X).
//
// Produces the same container sections as the host encoder, from elements
// already in device memory.  The pages encode offline and describe no
// encoder kernel; the format it fills is the one the DFloat11 digest
// ("DFloat11: compressao sem perda para inferencia em GPU...", sections
// "O formato DFloat11" and "Kernel de GPU em 2 etapas e metadados
// auxiliares") describes: codes concatenated into one stream, a 5-bit gap
// per 64-bit chunk (where its first code starts), one output index per
// 16384-bit tile, and for BF16 the packed sign|mantissa bytes.
//
// Each element's code starts at the sum of the lengths of the codes before
// it.  That sum is a scan over the elements, done in three launches:
//   enc_sums   one workgroup per block of kBlock elements sums its lengths;
//   enc_scan_local, enc_scan_add   the block sums into block start bits;
//   enc_write  each workgroup rescans its block, packs its codes into an
//              LDS bit buffer and writes it out (interior words with plain
//              stores; the first and last words, shared with the
//              neighbouring blocks, with atomic ORs into the zeroed stream),
//              and writes the gap field of every chunk and the offset of
//              every tile in which one of its codes is the first to start.
// enc_finish then writes tile_out[n_tiles] = n and the largest tile.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>

#include "dfh.h"

// Workspace of df_encode_device_noalloc, in the library's code object: each
// device the library runs on holds its own copy until the process ends.
// Host code never uses this name as an address (on the host it is only a
// stand-in for the symbol); it takes each device's address once with
// hipGetSymbolAddress and passes that to the kernels.
static __device__ __align__(256) uint8_t scratch[DF_ENCODE_SCRATCH_BYTES];

namespace {

constexpr uint32_t kThreads = 256;                 // encoder workgroup
constexpr uint32_t kPerThread = 16;                // consecutive elements per thread
constexpr uint32_t kBlock = kThreads * kPerThread;  // elements per block
constexpr uint32_t kGapBits = 5;

struct Codebook {
  uint32_t rev[256];  // code with its first bit at bit 0 (stream order)
  uint8_t len[256];   // 0 = no code
};

__device__ __forceinline__ uint32_t symbol_at(int kind, const void *src, uint64_t i) {
  if (kind == DF_KIND_BF16) return (((const uint16_t *)src)[i] >> 7) & 0xFFu;
  if (kind == DF_KIND_U4) return (((const uint8_t *)src)[i >> 1] >> (4 * (uint32_t)(i & 1))) & 0xFu;
  return ((const uint8_t *)src)[i];
}

// The raw bytes of elements i0 .. i0 + kPerThread - 1 (all below n), with
// 16-byte loads (i0 is a multiple of kPerThread, so they are aligned): 32
// bytes for BF16, 16 for uint8, 8 for uint4.
__device__ __forceinline__ void load16(int kind, const void *src, uint64_t i0, uint4 &a, uint4 &b) {
  if (kind == DF_KIND_BF16) {
    const uint4 *p = (const uint4 *)((const uint16_t *)src + i0);
    a = p[0];
    b = p[1];
  } else if (kind == DF_KIND_U8) {
    a = *(const uint4 *)((const uint8_t *)src + i0);
  } else {
    const uint2 v = *(const uint2 *)((const uint8_t *)src + i0 / 2);
    a = make_uint4(v.x, v.y, 0u, 0u);
  }
}

// Their symbols.
__device__ __forceinline__ void extract16(int kind, const uint4 &a, const uint4 &b, uint32_t (&s)[kPerThread]) {
  if (kind == DF_KIND_BF16) {
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (uint32_t k = 0; k < 8; k++) {
      s[2 * k] = (w[k] >> 7) & 0xFFu;
      s[2 * k + 1] = (w[k] >> 23) & 0xFFu;
    }
  } else if (kind == DF_KIND_U8) {
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (uint32_t k = 0; k < 16; k++) s[k] = (w[k >> 2] >> (8 * (k & 3))) & 0xFFu;
  } else {
    const uint32_t w[2] = {a.x, a.y};
#pragma unroll
    for (uint32_t k = 0; k < 16; k++) s[k] = (w[k >> 3] >> (4 * (k & 7))) & 0xFu;
  }
}

__device__ __forceinline__ void symbols16(int kind, const void *src, uint64_t i0, uint32_t (&s)[kPerThread]) {
  uint4 a = make_uint4(0u, 0u, 0u, 0u), b = a;
  load16(kind, src, i0, a, b);
  extract16(kind, a, b, s);
}

__global__ void fill_zero(uint32_t *p, uint64_t words) {
  for (uint64_t i = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; i < words;
       i += (uint64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

// Sixteen 256-bin LDS histograms per workgroup, four per wave chosen by
// lane, so few lanes add to one bin at a time (coded symbols crowd into a
// few bins); each padded to 257 words so that one bin of different copies
// sits in different banks.  16 consecutive elements per thread per step.
constexpr uint32_t kSubHists = 16, kSubStride = 257;
__global__ __launch_bounds__(kThreads) void histogram_kernel(int kind, const void *src, uint64_t n,
                                                             unsigned long long *hist) {
  __shared__ uint32_t h[kSubHists * kSubStride];
  for (uint32_t k = threadIdx.x; k < kSubHists * kSubStride; k += kThreads) h[k] = 0;
  __syncthreads();
  uint32_t *hw = h + ((threadIdx.x >> 6) * 4 + (threadIdx.x & 3)) * kSubStride;
  const uint64_t chunks = (n + kPerThread - 1) / kPerThread;
  for (uint64_t c = blockIdx.x * (uint64_t)kThreads + threadIdx.x; c < chunks; c += (uint64_t)gridDim.x * kThreads) {
    const uint64_t i0 = c * kPerThread;
    if (i0 + kPerThread <= n) {
      uint32_t sy[kPerThread];
      symbols16(kind, src, i0, sy);
#pragma unroll
      for (uint32_t k = 0; k < kPerThread; k++) atomicAdd(&hw[sy[k]], 1u);
    } else {
      for (uint64_t i = i0; i < n; i++) atomicAdd(&hw[symbol_at(kind, src, i)], 1u);
    }
  }
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (uint32_t j = 0; j < kSubHists; j++) t += h[j * kSubStride + threadIdx.x];
  if (t) atomicAdd(&hist[threadIdx.x], (unsigned long long)t);
}

// Sum of the workgroup's 256 values, returned to every thread.
__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t *scratch) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
  __syncthreads();
  const uint32_t s = scratch[0] + scratch[1] + scratch[2] + scratch[3];
  __syncthreads();
  return s;
}

// Exclusive prefix sum of the workgroup's 256 values in thread order.
__device__ __forceinline__ uint32_t block_exclusive(uint32_t v, uint32_t *scratch) {
  const uint32_t lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t x = v;
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= (uint32_t)o) x += y;
  }
  if (lane == 63) scratch[w] = x;
  __syncthreads();
  uint32_t before = 0;
  for (uint32_t k = 0; k < w; k++) before += scratch[k];
  __syncthreads();
  return before + x - v;
}

__global__ __launch_bounds__(kThreads) void enc_sums(int kind, const void *src, uint64_t n, Codebook cb,
                                                     uint64_t *block_sums) {
  __shared__ uint8_t len[256];
  __shared__ uint32_t scratch[4];
  len[threadIdx.x] = cb.len[threadIdx.x];
  __syncthreads();
  const uint64_t i0 = (uint64_t)blockIdx.x * kBlock + (uint64_t)threadIdx.x * kPerThread;
  uint32_t s = 0;
  if (i0 + kPerThread <= n) {
    uint32_t sy[kPerThread];
    symbols16(kind, src, i0, sy);
#pragma unroll
    for (uint32_t k = 0; k < kPerThread; k++) s += len[sy[k]];
  } else {
    for (uint64_t i = i0; i < n; i++) s += len[symbol_at(kind, src, i)];
  }
  s = block_sum(s, scratch);
  if (threadIdx.x == 0) block_sums[blockIdx.x] = s;
}

// block_base[b] = sum of block_sums[0 .. b), in two launches over
// segments of 1024 blocks: enc_scan_local scans each segment (coalesced) and
// records its total; enc_scan_add adds the totals of the segments before.
__global__ __launch_bounds__(1024) void enc_scan_local(const uint64_t *block_sums, uint64_t nblocks,
                                                       uint64_t *block_base, uint64_t *seg_total) {
  __shared__ uint64_t part[16];
  const uint64_t i = blockIdx.x * 1024ull + threadIdx.x;
  const uint64_t v = i < nblocks ? block_sums[i] : 0;
  const uint32_t lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint64_t x = v;  // inclusive within the wave
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t y = __shfl_up(x, o);
    if (lane >= (uint32_t)o) x += y;
  }
  if (lane == 63) part[wv] = x;
  __syncthreads();
  uint64_t before = 0;
  for (uint32_t k = 0; k < wv; k++) before += part[k];
  if (i < nblocks) block_base[i] = before + x - v;
  if (threadIdx.x == 1023) seg_total[blockIdx.x] = before + x;
}

__global__ __launch_bounds__(1024) void enc_scan_add(uint64_t *block_base, uint64_t nblocks,
                                                     const uint64_t *seg_total) {
  __shared__ uint64_t pre;
  if (threadIdx.x < 64) {
    uint64_t t = 0;
    for (uint32_t k = threadIdx.x; k < blockIdx.x; k += 64) t += seg_total[k];
    for (int o = 32; o >= 1; o >>= 1) t += __shfl_xor(t, o);
    if (threadIdx.x == 0) pre = t;
  }
  __syncthreads();
  const uint64_t i = blockIdx.x * 1024ull + threadIdx.x;
  if (i < nblocks) block_base[i] += pre;
}

__global__ __launch_bounds__(kThreads) void enc_write(int kind, const void *src, uint64_t n, Codebook cb,
                                                      const uint64_t *block_base, uint32_t *bits,
                                                      uint32_t *gaps, uint64_t *tile_out, uint8_t *sm) {
  __shared__ uint32_t rev[256];
  __shared__ uint8_t len[256];
  __shared__ uint32_t scratch[4];
  // the block's codes, from the word its first bit falls in: at most
  // kBlock * 32 bits starting up to 31 bits into word 0, so words 0..kBlock
  __shared__ uint32_t buf[kBlock + 1];
  // the gap fields of the chunks whose first code is in this block, from
  // the gap word of the block's first chunk: at most kBlock * 32 / 64
  // chunks plus the partial ones at both ends
  constexpr uint32_t kGapWords = ((kBlock * 32 / 64 + 2) * kGapBits) / 32 + 4;
  __shared__ uint32_t gbuf[kGapWords];
  // the element loads, the block's first bit and the element before this
  // thread's first go in flight first, so their latency overlaps the
  // codebook staging below
  const uint64_t b0 = (uint64_t)blockIdx.x * kBlock;
  const uint64_t i0 = b0 + (uint64_t)threadIdx.x * kPerThread;  // this thread's first element
  const bool full = i0 + kPerThread <= n;
  uint4 ra = make_uint4(0u, 0u, 0u, 0u), rb = ra;
  if (full) load16(kind, src, i0, ra, rb);
  const uint64_t base = block_base[blockIdx.x];
  const uint32_t prev_sym = i0 > 0 && i0 < n ? symbol_at(kind, src, i0 - 1) : 0u;
  rev[threadIdx.x] = cb.rev[threadIdx.x];
  len[threadIdx.x] = cb.len[threadIdx.x];
  for (uint32_t k = threadIdx.x; k < kBlock + 1; k += kThreads) buf[k] = 0;
  for (uint32_t k = threadIdx.x; k < kGapWords; k += kThreads) gbuf[k] = 0;
  __syncthreads();

  uint32_t syms[kPerThread];
  uint32_t mine = 0;
  if (full) {
    extract16(kind, ra, rb, syms);
  } else {
#pragma unroll
    for (uint32_t k = 0; k < kPerThread; k++) syms[k] = i0 + k < n ? symbol_at(kind, src, i0 + k) : 0u;
  }
#pragma unroll
  for (uint32_t k = 0; k < kPerThread; k++) mine += i0 + k < n ? len[syms[k]] : 0u;
  const uint64_t word0 = base >> 5;  // global word of the block's first bit
  const uint64_t gword0 = ((base >> 6) * kGapBits) >> 5;  // global gap word of its first chunk
  uint64_t pos = base + block_exclusive(mine, scratch);
  // positions relative to a tile-aligned origin at or below the block's
  // first bit fit 32 bits and keep chunk and tile boundaries aligned; the
  // start of the element before this thread's first one may lie below it
  const uint64_t org = base & ~(uint64_t)(DF_TILE_BITS - 1);
  int32_t lpos = (int32_t)(pos - org);
  // gap bit of the chunk holding local position p, relative to gbuf:
  // (p >> 6) * kGapBits + gdelta, with gdelta in (-1312, 32): 32-bit math
  const int32_t gdelta = (int32_t)((org >> 6) * kGapBits - (gword0 << 5));
  int32_t lprev = i0 > 0 && i0 < n ? lpos - (int32_t)len[prev_sym] : lpos;
  const uint32_t count = full ? kPerThread : i0 < n ? (uint32_t)(n - i0) : 0u;

  // the thread's codes are packed in a register and whole words ORed into
  // the block buffer (its first and last word are shared with neighbours)
  const uint64_t lp0 = pos - (word0 << 5);
  uint32_t wix = (uint32_t)(lp0 >> 5), acc_bits = (uint32_t)(lp0 & 31);
  uint64_t acc = 0;
  // kept rolled: unrolled, the kernel needs 76 registers instead of 48 and
  // ran 8% slower
  for (uint32_t k = 0; k < count; k++) {
    const uint32_t s = syms[k], l = len[s];
    if (k == 0 && i0 == 0) {
      tile_out[0] = 0;  // gap field 0 is 0: the stream is cleared beforehand
    } else {
      if ((lprev >> 6) != (lpos >> 6)) {  // first code of its chunk
        const uint32_t at = (uint32_t)((lpos >> 6) * (int32_t)kGapBits + gdelta);
        const uint32_t g = (uint32_t)lpos & 63u, sh = at & 31;
        atomicOr(&gbuf[at >> 5], g << sh);
        if (sh > 32 - kGapBits) atomicOr(&gbuf[(at >> 5) + 1], g >> (32 - sh));
        if ((lprev >> 14) != (lpos >> 14))  // first code of its tile (a tile starts a chunk)
          tile_out[(org >> 14) + (uint64_t)(lpos >> 14)] = i0 + k;
      }
    }
    // the code's bits after the accumulated ones (acc_bits < 32, l <= 32)
    acc |= (uint64_t)rev[s] << acc_bits;
    acc_bits += l;
    if (acc_bits >= 32) {  // (a zero word ORs nothing: no test for it)
      atomicOr(&buf[wix], (uint32_t)acc);
      acc >>= 32;
      acc_bits -= 32;
      wix++;
    }
    lprev = lpos;
    lpos += (int32_t)l;
  }
  if (acc_bits && (uint32_t)acc) atomicOr(&buf[wix], (uint32_t)acc);
  if (kind == DF_KIND_BF16) {  // sign|mantissa bytes of this thread's elements
    const uint16_t *u = (const uint16_t *)src;
    if (full) {  // from the words already loaded: two elements per word
      const uint32_t w[8] = {ra.x, ra.y, ra.z, ra.w, rb.x, rb.y, rb.z, rb.w};
      uint32_t o[kPerThread / 4];
#pragma unroll
      for (uint32_t q = 0; q < kPerThread / 4; q++) {
        uint32_t x = 0;
#pragma unroll
        for (uint32_t r = 0; r < 4; r++) {
          const uint32_t e = (w[2 * q + (r >> 1)] >> (16 * (r & 1))) & 0xFFFFu;
          x |= (((e >> 8) & 0x80u) | (e & 0x7Fu)) << (8 * r);
        }
        o[q] = x;
      }
      *(uint4 *)(sm + i0) = make_uint4(o[0], o[1], o[2], o[3]);
    } else {
      for (uint64_t i = i0; i < n; i++) sm[i] = (uint8_t)(((u[i] >> 8) & 0x80u) | (u[i] & 0x7Fu));
    }
  }
  __syncthreads();

  // out: the block's bit range [base, base + its lengths) as words word0 ..
  const uint64_t last_bit = base + block_sum(mine, scratch);
  if (last_bit == base) return;
  const uint64_t nwords = ((last_bit + 31) >> 5) - word0;
  for (uint64_t k = threadIdx.x; k < nwords; k += kThreads) {
    const uint32_t v = buf[k];
    const bool edge = k == 0 || k == nwords - 1;  // shared with the block before or after
    if (edge) {
      if (v) atomicOr(&bits[word0 + k], v);
    } else {
      bits[word0 + k] = v;
    }
  }
  // gap words: a field can straddle two words, so the first two and the last
  // two may hold fields written by the neighbouring blocks
  const uint64_t ngw = ((((last_bit - 1) >> 6) * kGapBits + kGapBits - 1) >> 5) - gword0 + 1;
  for (uint64_t k = threadIdx.x; k < ngw; k += kThreads) {
    const uint32_t v = gbuf[k];
    if (k < 2 || k + 2 >= ngw) {
      if (v) atomicOr(&gaps[gword0 + k], v);
    } else {
      gaps[gword0 + k] = v;
    }
  }
}

// The coded symbol of element i, for the host's layout call.
__global__ void symbol_kernel(int kind, const void *src, uint64_t i, uint64_t *out) {
  if (threadIdx.x == 0) *out = symbol_at(kind, src, i);
}

__global__ void enc_finish(uint64_t *tile_out, uint64_t n_tiles, uint64_t n, uint32_t *max_tile) {
  for (uint64_t b = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; b < n_tiles;
       b += (uint64_t)gridDim.x * blockDim.x) {
    const uint64_t hi = b + 1 == n_tiles ? n : tile_out[b + 1];
    atomicMax(max_tile, (uint32_t)(hi - tile_out[b]));
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) tile_out[n_tiles] = n;
}

uint64_t blocks_for(uint64_t n) { return (n + kBlock - 1) / kBlock; }
uint64_t segments_for(uint64_t nblocks) { return (nblocks + 1023) / 1024; }

}  // namespace

extern "C" {

uint64_t df_encode_workspace_bytes(uint64_t n) {
  // block sums, block bases, segment totals
  return 8 * (2 * (blocks_for(n) + 1) + segments_for(blocks_for(n)) + 1) + 16;
}

df_status df_histogram_device(df_kind kind, const void *d_src, uint64_t n, uint64_t *d_hist,
                              hipStream_t stream) {
  if (!d_hist || (n && (!d_src || ((uintptr_t)d_src & 15))) ||
      (kind != DF_KIND_BF16 && kind != DF_KIND_U8 && kind != DF_KIND_U4))
    return DF_ERR_ARG;
  hipLaunchKernelGGL(fill_zero, dim3(1), dim3(256), 0, stream, (uint32_t *)d_hist, (uint64_t)512);
  if (n) {
    uint64_t grid = (n + kThreads * kPerThread * 8 - 1) / (kThreads * kPerThread * 8);
    if (grid > 2048) grid = 2048;
    hipLaunchKernelGGL(histogram_kernel, dim3((uint32_t)grid), dim3(kThreads), 0, stream, (int)kind, d_src, n,
                       (unsigned long long *)d_hist);
  }
  return hipGetLastError() == hipSuccess ? DF_OK : DF_ERR_HIP;
}

df_status df_symbol_device(df_kind kind, const void *d_src, uint64_t i, uint64_t *d_sym, hipStream_t stream) {
  if (!d_src || !d_sym || ((uintptr_t)d_sym & 7) ||
      (kind != DF_KIND_BF16 && kind != DF_KIND_U8 && kind != DF_KIND_U4))
    return DF_ERR_ARG;
  hipLaunchKernelGGL(symbol_kernel, dim3(1), dim3(64), 0, stream, (int)kind, d_src, i, d_sym);
  return hipGetLastError() == hipSuccess ? DF_OK : DF_ERR_HIP;
}

}  // extern "C"

namespace {

// The device address of `scratch` on each device, taken once per device.
constexpr int kMaxDevices = 64;
void *g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

df_status scratch_address(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DF_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DF_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return DF_OK;
}

df_status encode_device(df_kind kind, const void *d_src, uint64_t n, const uint8_t lengths[256],
                        const df_info *layout, uint8_t *d_bitstream, uint8_t *d_gaps, uint64_t *d_tile_out,
                        uint8_t *d_sign_mantissa, void *d_workspace, uint32_t *d_max_tile, hipStream_t stream);

}  // namespace

extern "C" {

df_status df_encode_device(df_kind kind, const void *d_src, uint64_t n, const uint8_t lengths[256],
                           const df_info *layout, uint8_t *d_bitstream, uint8_t *d_gaps,
                           uint64_t *d_tile_out, uint8_t *d_sign_mantissa, void *d_workspace,
                           uint32_t *d_max_tile, hipStream_t stream) {
  if (n && (!d_workspace || ((uintptr_t)d_workspace & 15))) return DF_ERR_ARG;
  return encode_device(kind, d_src, n, lengths, layout, d_bitstream, d_gaps, d_tile_out, d_sign_mantissa,
                       d_workspace, d_max_tile, stream);
}

df_status df_encode_device_noalloc(df_kind kind, const void *d_src, uint64_t n, const uint8_t lengths[256],
                                   const df_info *layout, uint8_t *d_bitstream, uint8_t *d_gaps,
                                   uint64_t *d_tile_out, uint8_t *d_sign_mantissa, uint32_t *d_max_tile,
                                   hipStream_t stream) {
  if (df_encode_workspace_bytes(n) > DF_ENCODE_SCRATCH_BYTES) return DF_ERR_ARG;
  void *ws = nullptr;
  const df_status st = scratch_address(&ws);
  if (st != DF_OK) return st;
  return encode_device(kind, d_src, n, lengths, layout, d_bitstream, d_gaps, d_tile_out, d_sign_mantissa, ws,
                       d_max_tile, stream);
}

}  // extern "C"

namespace {

df_status encode_device(df_kind kind, const void *d_src, uint64_t n, const uint8_t lengths[256],
                        const df_info *layout, uint8_t *d_bitstream, uint8_t *d_gaps, uint64_t *d_tile_out,
                        uint8_t *d_sign_mantissa, void *d_workspace, uint32_t *d_max_tile, hipStream_t stream) {
  if (!lengths || !layout || (kind != DF_KIND_BF16 && kind != DF_KIND_U8 && kind != DF_KIND_U4) ||
      layout->kind != kind || layout->n != n || !d_tile_out || !d_max_tile)
    return DF_ERR_ARG;
  if (n && (!d_src || ((uintptr_t)d_src & 15) || !d_bitstream || !d_gaps || !d_workspace ||
            ((uintptr_t)d_workspace & 15) || ((uintptr_t)d_bitstream & 15) || ((uintptr_t)d_gaps & 15) ||
            ((uintptr_t)d_tile_out & 7)))
    return DF_ERR_ARG;
  if (kind == DF_KIND_BF16 && n && (!d_sign_mantissa || ((uintptr_t)d_sign_mantissa & 15))) return DF_ERR_ARG;
  if (memcmp(layout->lengths, lengths, 256) != 0) return DF_ERR_ARG;
  // the canonical code of every length (RFC 1951 3.2.2), bit-reversed into
  // stream order
  Codebook cb;
  memset(&cb, 0, sizeof cb);
  {
    uint32_t count[DF_MAX_LEN + 2] = {0}, next[DF_MAX_LEN + 2] = {0};
    for (int s = 0; s < 256; s++)
      if (lengths[s]) {
        if (lengths[s] > DF_MAX_LEN) return DF_ERR_CODEBOOK;
        count[lengths[s]]++;
      }
    uint64_t code = 0;
    for (int l = 1; l <= DF_MAX_LEN; l++) {
      code = (code + count[l - 1]) << 1;
      next[l] = (uint32_t)code;
    }
    for (int s = 0; s < 256; s++) {
      const uint32_t l = lengths[s];
      cb.len[s] = (uint8_t)l;
      if (!l) continue;
      const uint32_t c = next[l]++;
      uint32_t r = 0;
      for (uint32_t k = 0; k < l; k++) r |= ((c >> (l - 1 - k)) & 1u) << k;
      cb.rev[s] = r;
    }
  }
  const uint64_t n_tiles = layout->n_tiles;
  hipLaunchKernelGGL(fill_zero, dim3(1), dim3(32), 0, stream, d_max_tile, (uint64_t)1);
  // the stream and gap sections are ORed into, so they start zero; their
  // padding (the whole section when n == 0) stays zero
  const uint64_t zb = layout->section_bytes[DF_SEC_BITSTREAM] / 4, zg = layout->section_bytes[DF_SEC_GAPS] / 4;
  if (d_bitstream && zb) hipLaunchKernelGGL(fill_zero, dim3(1024), dim3(256), 0, stream, (uint32_t *)d_bitstream, zb);
  if (d_gaps && zg) hipLaunchKernelGGL(fill_zero, dim3(64), dim3(256), 0, stream, (uint32_t *)d_gaps, zg);
  if (kind == DF_KIND_BF16 && d_sign_mantissa) {  // the padding past n
    const uint64_t pad0 = n & ~(uint64_t)63, words = (layout->section_bytes[DF_SEC_SIGN_MANTISSA] - pad0) / 4;
    if (words)
      hipLaunchKernelGGL(fill_zero, dim3(1), dim3(64), 0, stream, (uint32_t *)(d_sign_mantissa + pad0), words);
  }
  if (n == 0) {
    hipLaunchKernelGGL(enc_finish, dim3(1), dim3(64), 0, stream, d_tile_out, (uint64_t)0, (uint64_t)0,
                       d_max_tile);
    return hipGetLastError() == hipSuccess ? DF_OK : DF_ERR_HIP;
  }
  const uint64_t nb = blocks_for(n);
  if (nb > 0xFFFFFFFFull) return DF_ERR_ARG;
  uint64_t *sums = (uint64_t *)d_workspace, *bases = sums + nb + 1, *segs = bases + nb + 1;
  const uint64_t nseg = segments_for(nb);
  hipLaunchKernelGGL(enc_sums, dim3((uint32_t)nb), dim3(kThreads), 0, stream, (int)kind, d_src, n, cb, sums);
  hipLaunchKernelGGL(enc_scan_local, dim3((uint32_t)nseg), dim3(1024), 0, stream, (const uint64_t *)sums, nb, bases,
                     segs);
  hipLaunchKernelGGL(enc_scan_add, dim3((uint32_t)nseg), dim3(1024), 0, stream, bases, nb, (const uint64_t *)segs);
  hipLaunchKernelGGL(enc_write, dim3((uint32_t)nb), dim3(kThreads), 0, stream, (int)kind, d_src, n, cb,
                     (const uint64_t *)bases, (uint32_t *)d_bitstream, (uint32_t *)d_gaps, d_tile_out,
                     d_sign_mantissa);
  uint64_t grid = (n_tiles + 255) / 256;
  if (grid < 1) grid = 1;
  if (grid > 1024) grid = 1024;
  hipLaunchKernelGGL(enc_finish, dim3((uint32_t)grid), dim3(256), 0, stream, d_tile_out, n_tiles, n, d_max_tile);
  return hipGetLastError() == hipSuccess ? DF_OK : DF_ERR_HIP;
}

}  // namespace
