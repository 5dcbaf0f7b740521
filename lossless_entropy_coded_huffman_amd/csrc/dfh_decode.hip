// dfh_decode.hip -- gfx950 decompression kernels and the device half of the
// C ABI (include/dfh.h).
//
// The DFloat11 digest ("DFloat11: compressao sem perda para inferencia em
// GPU que reduz LLMs para 70% do tamanho"), section "Kernel de GPU em 2
// etapas e metadados auxiliares": every thread owns 8 bytes of the encoded
// stream and decodes the codes that start inside them; the Gaps array says
// where its first code starts; only the first output index of each thread
// block is stored; phase 1 decodes and counts without writing memory, a
// prefix sum over the block gives each thread its output index, phase 2
// decodes again into an on-chip buffer, and one coalesced pass writes the
// block's output.  Section "Decodificacao com LUT hierarquica": code tables
// live in on-chip memory.  Section "Descompressao por bloco de transformer":
// a whole block of matrices is one launch.
//
// The gfx950 design (one workgroup = 256 lanes = 4 wave64):
//   - persistent workgroups: each stages its container's tables in LDS once
//     (the 4096-entry multi-code table, 32 KiB, and the hierarchical tables,
//     512 B each) and then loops over tiles;
//   - a lane keeps its 8 stream bytes plus the next 4 in three registers
//     (12-byte window) loaded straight from HBM, so the stream is read once;
//   - a lookup in the multi-code table yields up to five codes; codes longer
//     than 12 bits fall back to the hierarchical tables;
//   - the block prefix sum is a wave64 DPP scan (row_shr, row_bcast) plus one
//     LDS step across the four waves;
//   - phase 2 ORs the decoded bytes into an LDS staging buffer laid out so
//     that its byte j holds output element (tile start rounded down to the
//     16-byte store granule) + j; the store pass then reads aligned LDS
//     words, merges the sign|mantissa bytes (BF16) and issues 16-byte
//     global stores.

#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>

#include "dfh.h"

namespace {

constexpr uint32_t kTPB = DF_THREADS_PER_TILE;  // lanes per workgroup = threads per tile
constexpr uint32_t kK = DF_DTAB_BITS;           // multi-code table index width
constexpr uint32_t kDtabEntries = 1u << kK;
constexpr uint32_t kDtabBytes = kDtabEntries * 8;

struct Job {
  const uint32_t *bits;  // bitstream, little-endian 32-bit words
  const uint32_t *gaps;  // packed 5-bit gaps as 32-bit words
  const uint64_t *tile_out;
  const uint8_t *sm;
  const uint16_t *lut;
  const uint64_t *dtab;
  void *dst;
  uint64_t n, total_bits, n_threads, n_tiles;
  uint32_t n_luts, wg_begin, wg_count, max_tile_elems;
};

struct Batch {
  Job job[DF_MAX_BATCH];
  uint32_t count;
  uint32_t lds_out_bytes;  // output staging area at the start of LDS
  uint32_t *err;           // error word (checked launches only)
};

// Stream bits [p, p + 32) of the 96-bit window w2:w1:w0, for p < 64.
__device__ __forceinline__ uint32_t window(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t p) {
  const bool up = p >= 32;
  const uint32_t lo = up ? w1 : w0;
  const uint32_t hi = up ? w2 : w1;
  return (uint32_t)((((uint64_t)hi << 32) | lo) >> (p & 31));
}

// One code through the hierarchical tables: returns (length << 8) | symbol.
// A prefix with no code (possible only for an incomplete code or a corrupt
// stream) reports DF_DEVERR_CODE in checked launches and consumes one bit.
template <bool CHECKED>
__device__ __forceinline__ uint32_t long_code(const uint16_t *lut, uint32_t n_luts, uint32_t win,
                                           uint32_t *err) {
  uint32_t e = lut[win & 255];
  uint32_t sh = 8;
  for (int d = 0; d < 3 && (e & 0x8000u); d++) {
    const uint32_t t = e & 0x7FFFu;
    if (t >= n_luts) break;
    e = lut[t * 256 + ((win >> sh) & 255)];
    sh += 8;
  }
  if ((e & 0x8000u) || (e >> 8) == 0) {
    if (CHECKED) atomicOr(err, DF_DEVERR_CODE);
    return 1u << 8;
  }
  return e;
}

__device__ __forceinline__ uint32_t rot_right1(uint32_t s) { return ((s >> 1) | (s << 7)) & 0xFFu; }

// Inclusive sum over the 64 lanes of a wave with DPP: shifts of 1, 2, 4, 8
// inside each 16-lane row, then row 0's last lane is added to row 1 and row
// 2's to row 3 (row_bcast:15), then lane 31 to rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false); // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false); // row_bcast:31
  return x;
}

// Exclusive prefix sum over the 256 lanes; *total gets the sum.  Contains a
// barrier.
__device__ __forceinline__ uint32_t block_exclusive_sum(uint32_t v, uint32_t *wsum, uint32_t *total) {
  const uint32_t lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint32_t x = wave_inclusive_sum(v);
  if (lane == 63) wsum[wid] = x;
  __syncthreads();
  const uint32_t s0 = wsum[0], s1 = wsum[1], s2 = wsum[2], s3 = wsum[3];
  *total = s0 + s1 + s2 + s3;
  const uint32_t before = (wid > 0 ? s0 : 0u) + (wid > 1 ? s1 : 0u) + (wid > 2 ? s2 : 0u);
  return before + x - v;
}

// OR up to five symbol bytes (s0 = bytes 0..3, s1 = byte 4) into the staging
// buffer at byte q; they span at most two aligned words.
__device__ __forceinline__ void put_bytes(uint8_t *out, uint32_t q, uint32_t qmax, uint32_t s0,
                                          uint32_t s1) {
  const uint32_t qq = q < qmax ? q : qmax;
  const uint64_t v = ((((uint64_t)s1) << 32) | s0) << ((qq & 3) * 8);
  uint32_t *w = (uint32_t *)(out + (qq & ~3u));
  atomicOr(w, (uint32_t)v);
  atomicOr(w + 1, (uint32_t)(v >> 32));
}

// Merge four exponent bytes (rotated right by one bit) with four
// sign|mantissa bytes into four BF16 values (two words):
// BF16 low byte = e0 << 7 | mantissa, high byte = sign << 7 | e >> 1.
__device__ __forceinline__ uint2 merge4(uint32_t e4, uint32_t s4) {
  const uint32_t x0 = __builtin_amdgcn_perm(e4, s4, 0x05010400u);  // s0 e0 s1 e1
  const uint32_t y0 = __builtin_amdgcn_perm(e4, s4, 0x01050004u);  // e0 s0 e1 s1
  const uint32_t x1 = __builtin_amdgcn_perm(e4, s4, 0x07030602u);  // s2 e2 s3 e3
  const uint32_t y1 = __builtin_amdgcn_perm(e4, s4, 0x03070206u);  // e2 s2 e3 s3
  return make_uint2((x0 & 0x7F7F7F7Fu) | (y0 & 0x80808080u), (x1 & 0x7F7F7F7Fu) | (y1 & 0x80808080u));
}

template <int KIND, bool CHECKED>
__global__ __launch_bounds__(256) void decode_kernel(const Batch batch) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ uint32_t wsum[4];

  const uint32_t wg = blockIdx.x;
  uint32_t j = 0;
  while (j + 1 < batch.count && wg >= batch.job[j + 1].wg_begin) j++;
  const Job &jb = batch.job[j];
  const uint32_t tid = threadIdx.x;

  uint8_t *out_lds = smem;
  const uint32_t lds_out_bytes = batch.lds_out_bytes;
  uint64_t *dtab_lds = (uint64_t *)(smem + lds_out_bytes);
  uint16_t *lut_lds = (uint16_t *)(smem + lds_out_bytes + kDtabBytes);
  const uint32_t n_luts = jb.n_luts;

  {  // stage the tables once per workgroup
    const uint4 *src = (const uint4 *)jb.dtab;
    uint4 *dl = (uint4 *)dtab_lds;
    for (uint32_t i = tid; i < kDtabBytes / 16; i += kTPB) dl[i] = src[i];
    const uint4 *ls = (const uint4 *)jb.lut;
    uint4 *ll = (uint4 *)lut_lds;
    for (uint32_t i = tid; i < n_luts * 32; i += kTPB) ll[i] = ls[i];
  }
  __syncthreads();

  const uint32_t *dtab_words = (const uint32_t *)dtab_lds;
  const uint32_t qmax = lds_out_bytes - 8;

  for (uint64_t tile = wg - jb.wg_begin; tile < jb.n_tiles; tile += jb.wg_count) {
    uint64_t lo = jb.tile_out[tile];
    uint64_t hi = jb.tile_out[tile + 1];
    if (hi > jb.n) hi = jb.n;
    if (lo > hi) lo = hi;
    if (hi - lo > jb.max_tile_elems) hi = lo + jb.max_tile_elems;
    const uint64_t a = KIND == DF_KIND_BF16 ? (lo & ~7ull) : (lo & ~15ull);

    // this lane's chunk: stream bits [64T, 64T + 96) and its gap
    const uint64_t T = tile * kTPB + tid;
    const uint2 w01 = *(const uint2 *)(jb.bits + 2 * T);
    const uint32_t w0 = w01.x, w1 = w01.y, w2 = jb.bits[2 * T + 2];
    uint32_t gap = 0, E = 0;
    if (T < jb.n_threads) {
      const uint64_t gb = 5 * T;
      const uint32_t g0 = jb.gaps[gb >> 5], g1 = jb.gaps[(gb >> 5) + 1];
      gap = (uint32_t)(((((uint64_t)g1) << 32) | g0) >> (gb & 31)) & 31u;
      const uint64_t rem = jb.total_bits - 64 * T;
      E = rem < 64 ? (uint32_t)rem : 64u;
    }

    // clear the staging bytes this tile uses (plus the spill word)
    const uint32_t span = (uint32_t)(hi - a);
    const uint32_t zero_bytes = (span + 8 + 15) & ~15u;
    for (uint32_t i = tid * 16; i < zero_bytes; i += kTPB * 16)
      *(uint4 *)(out_lds + i) = make_uint4(0, 0, 0, 0);

    // phase 1: count the codes that start in [gap, E)
    uint32_t cnt = 0;
    {
      uint32_t p = gap;
      while (p + kK < E) {
        const uint32_t win = window(w0, w1, w2, p);
        const uint32_t h = dtab_words[2 * (win & (kDtabEntries - 1)) + 1];
        uint32_t adv = (h >> 24) & 15;
        uint32_t nc = h >> 28;
        if (adv == 0) {
          adv = long_code<CHECKED>(lut_lds, n_luts, win, batch.err) >> 8;
          nc = 1;
        }
        cnt += nc;
        p += adv;
      }
      while (p < E) {
        const uint32_t win = window(w0, w1, w2, p);
        const uint32_t h = dtab_words[2 * (win & (kDtabEntries - 1)) + 1];
        uint32_t adv = (h >> 24) & 15;
        uint32_t starts = (h >> 8) & 0xFFFu;
        if (adv == 0) {
          adv = long_code<CHECKED>(lut_lds, n_luts, win, batch.err) >> 8;
          starts = 1;
        }
        cnt += __popc(starts & ((1u << (E - p)) - 1));  // E - p <= 12 here
        p += adv;
      }
    }

    uint32_t total;
    const uint32_t off = block_exclusive_sum(cnt, wsum, &total);
    if (CHECKED && tid == 0 && (uint64_t)total != hi - lo) atomicOr(batch.err, DF_DEVERR_COUNT);

    // phase 2: decode again, OR the symbol bytes into the staging buffer
    {
      uint32_t p = gap;
      uint32_t q = (uint32_t)(lo - a) + off;
      while (p + kK < E) {
        const uint32_t win = window(w0, w1, w2, p);
        const uint2 e = *(const uint2 *)(dtab_lds + (win & (kDtabEntries - 1)));
        uint32_t adv = (e.y >> 24) & 15;
        uint32_t nc = e.y >> 28;
        uint32_t s0 = e.x, s1 = e.y & 0xFFu;
        if (adv == 0) {
          const uint32_t r = long_code<CHECKED>(lut_lds, n_luts, win, batch.err);
          adv = r >> 8;
          s0 = KIND == DF_KIND_BF16 ? rot_right1(r & 0xFFu) : (r & 0xFFu);
          s1 = 0;
          nc = 1;
        }
        put_bytes(out_lds, q, qmax, s0, s1);
        q += nc;
        p += adv;
      }
      while (p < E) {
        const uint32_t win = window(w0, w1, w2, p);
        const uint2 e = *(const uint2 *)(dtab_lds + (win & (kDtabEntries - 1)));
        uint32_t adv = (e.y >> 24) & 15;
        uint32_t starts = (e.y >> 8) & 0xFFFu;
        uint32_t s0 = e.x, s1 = e.y & 0xFFu;
        if (adv == 0) {
          const uint32_t r = long_code<CHECKED>(lut_lds, n_luts, win, batch.err);
          adv = r >> 8;
          s0 = KIND == DF_KIND_BF16 ? rot_right1(r & 0xFFu) : (r & 0xFFu);
          s1 = 0;
          starts = 1;
        }
        const uint32_t nc = __popc(starts & ((1u << (E - p)) - 1));
        if (nc < 5) {
          s1 = 0;
          if (nc < 4) s0 &= (1u << (8 * nc)) - 1;
        }
        put_bytes(out_lds, q, qmax, s0, s1);
        q += nc;
        p += adv;
      }
    }
    __syncthreads();

    // one coalesced pass: aligned 16-byte stores of the tile's output range
    if (KIND == DF_KIND_BF16) {
      uint16_t *dst = (uint16_t *)jb.dst;
      const uint32_t groups = (uint32_t)(((hi + 7) >> 3) - (lo >> 3));
      for (uint32_t g = tid; g < groups; g += kTPB) {
        const uint64_t e0 = a + 8ull * g;
        const uint2 ex = *(const uint2 *)(out_lds + 8 * g);
        const uint2 sv = *(const uint2 *)(jb.sm + e0);
        const uint2 o01 = merge4(ex.x, sv.x);
        const uint2 o23 = merge4(ex.y, sv.y);
        if (e0 >= lo && e0 + 8 <= hi) {
          *(uint4 *)(dst + e0) = make_uint4(o01.x, o01.y, o23.x, o23.y);
        } else {
          const uint32_t o[4] = {o01.x, o01.y, o23.x, o23.y};
          for (uint32_t k = 0; k < 8; k++)
            if (e0 + k >= lo && e0 + k < hi) dst[e0 + k] = (uint16_t)(o[k >> 1] >> (16 * (k & 1)));
        }
      }
    } else {
      uint8_t *dst = (uint8_t *)jb.dst;
      const uint32_t groups = (uint32_t)(((hi + 15) >> 4) - (lo >> 4));
      for (uint32_t g = tid; g < groups; g += kTPB) {
        const uint64_t e0 = a + 16ull * g;
        const uint4 v = *(const uint4 *)(out_lds + 16 * g);
        if (e0 >= lo && e0 + 16 <= hi) {
          *(uint4 *)(dst + e0) = v;
        } else {
          const uint32_t o[4] = {v.x, v.y, v.z, v.w};
          for (uint32_t k = 0; k < 16; k++)
            if (e0 + k >= lo && e0 + k < hi) dst[e0 + k] = (uint8_t)(o[k >> 2] >> (8 * (k & 3)));
        }
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ host side
struct DeviceProps {
  bool ready;
  int cus;
  int max_lds;
};
constexpr int kMaxDevices = 64;
DeviceProps g_props[kMaxDevices];
std::mutex g_mu;

typedef void (*KernelFn)(const Batch);
KernelFn kernel_for(df_kind kind, bool checked) {
  if (kind == DF_KIND_BF16) return checked ? decode_kernel<DF_KIND_BF16, true> : decode_kernel<DF_KIND_BF16, false>;
  return checked ? decode_kernel<DF_KIND_U8, true> : decode_kernel<DF_KIND_U8, false>;
}

df_status device_props(DeviceProps *out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DF_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_mu);
  DeviceProps &p = g_props[dev];
  if (!p.ready) {
    if (hipDeviceGetAttribute(&p.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipDeviceGetAttribute(&p.max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
      return DF_ERR_HIP;
    // allow dynamic LDS up to the device limit; where the runtime needs no
    // opt-in the call may fail, which is harmless, so its error is cleared
    const df_kind kinds[2] = {DF_KIND_BF16, DF_KIND_U8};
    for (df_kind k : kinds)
      for (int c = 0; c < 2; c++)
        if (hipFuncSetAttribute((const void *)kernel_for(k, c != 0),
                                hipFuncAttributeMaxDynamicSharedMemorySize, p.max_lds - 64) != hipSuccess)
          (void)hipGetLastError();
    p.ready = true;
  }
  *out = p;
  return DF_OK;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

df_status check_view(const df_device_view *v, const void *dst) {
  if (!v || (v->kind != DF_KIND_BF16 && v->kind != DF_KIND_U8)) return DF_ERR_ARG;
  if (v->n == 0) return DF_OK;
  if (!dst || !aligned(dst, 16)) return DF_ERR_ARG;
  if (!v->bitstream || !v->gaps || !v->tile_out || !v->lut || !v->dtab) return DF_ERR_ARG;
  if (v->kind == DF_KIND_BF16 && (!v->sign_mantissa || !aligned(v->sign_mantissa, 8))) return DF_ERR_ARG;
  if (!aligned(v->bitstream, 8) || !aligned(v->gaps, 4) || !aligned(v->tile_out, 8) ||
      !aligned(v->lut, 16) || !aligned(v->dtab, 16))
    return DF_ERR_ARG;
  if (v->n_tiles == 0 || v->n_threads == 0 || v->n_threads > v->n_tiles * DF_THREADS_PER_TILE ||
      v->n_threads <= (v->n_tiles - 1) * DF_THREADS_PER_TILE)
    return DF_ERR_ARG;
  if (v->total_bits <= (v->n_threads - 1) * 64 || v->total_bits > v->n_threads * 64 + DF_MAX_LEN)
    return DF_ERR_ARG;
  if (v->n_luts < 1 || v->n_luts > DF_MAX_LUTS) return DF_ERR_ARG;
  if (v->max_tile_elems < 1 || v->max_tile_elems > DF_TILE_BITS) return DF_ERR_ARG;
  return DF_OK;
}

uint32_t lds_out_bytes_for(uint32_t max_tile_elems) {
  // tile range rounded down to a 16-element granule, plus the 8-byte spill
  // of the last OR, rounded to 16, plus one spare granule
  return ((max_tile_elems + 15 + 8 + 15) & ~15u) + 16;
}

df_status launch(const df_device_view *views, void *const *dsts, uint32_t count, uint32_t *err,
                 bool checked, hipStream_t stream) {
  if (!views || !dsts) return DF_ERR_ARG;
  if (count == 0) return DF_OK;
  const df_kind kind = views[0].kind;
  for (uint32_t i = 0; i < count; i++) {
    df_status st = check_view(&views[i], dsts[i]);
    if (st != DF_OK) return st;
    if (views[i].kind != kind) return DF_ERR_ARG;
  }
  DeviceProps props;
  df_status st = device_props(&props);
  if (st != DF_OK) return st;
  KernelFn fn = kernel_for(kind, checked);

  for (uint32_t base = 0; base < count; base += DF_MAX_BATCH) {
    const uint32_t m = count - base < DF_MAX_BATCH ? count - base : DF_MAX_BATCH;
    Batch b;
    memset(&b, 0, sizeof b);
    uint32_t max_elems = 0, max_luts = 1;
    uint64_t tiles = 0;
    uint32_t nj = 0;
    uint32_t idx[DF_MAX_BATCH];
    for (uint32_t i = 0; i < m; i++) {
      const df_device_view &v = views[base + i];
      if (v.n == 0) continue;
      idx[nj++] = base + i;
      tiles += v.n_tiles;
      if (v.max_tile_elems > max_elems) max_elems = v.max_tile_elems;
      if (v.n_luts > max_luts) max_luts = v.n_luts;
    }
    if (nj == 0) continue;
    const uint32_t out_bytes = lds_out_bytes_for(max_elems);
    const size_t lds = (size_t)out_bytes + kDtabBytes + (size_t)max_luts * 512;
    if (lds > (size_t)props.max_lds) return DF_ERR_ARG;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void *)fn, (int)kTPB, lds) != hipSuccess)
      return DF_ERR_HIP;
    if (per_cu < 1) per_cu = 1;
    uint64_t budget = (uint64_t)props.cus * (uint64_t)per_cu;
    if (budget < nj) budget = nj;
    uint32_t wg = 0;
    for (uint32_t k = 0; k < nj; k++) {
      const df_device_view &v = views[idx[k]];
      uint64_t share = budget * v.n_tiles / tiles;
      if (share < 1) share = 1;
      if (share > v.n_tiles) share = v.n_tiles;
      Job &jb = b.job[k];
      jb.bits = (const uint32_t *)v.bitstream;
      jb.gaps = (const uint32_t *)v.gaps;
      jb.tile_out = v.tile_out;
      jb.sm = v.sign_mantissa;
      jb.lut = v.lut;
      jb.dtab = v.dtab;
      jb.dst = dsts[idx[k]];
      jb.n = v.n;
      jb.total_bits = v.total_bits;
      jb.n_threads = v.n_threads;
      jb.n_tiles = v.n_tiles;
      jb.n_luts = v.n_luts;
      jb.max_tile_elems = v.max_tile_elems;
      jb.wg_begin = wg;
      jb.wg_count = (uint32_t)share;
      wg += (uint32_t)share;
    }
    b.count = nj;
    b.lds_out_bytes = out_bytes;
    b.err = err;
    hipLaunchKernelGGL(fn, dim3(wg), dim3(kTPB), lds, stream, b);
    if (hipGetLastError() != hipSuccess) return DF_ERR_HIP;
  }
  return DF_OK;
}

}  // namespace

extern "C" {

df_status df_decompress(const df_device_view *v, void *dst, hipStream_t stream) {
  if (!v) return DF_ERR_ARG;
  void *d[1] = {dst};
  return launch(v, d, 1, nullptr, false, stream);
}

df_status df_decompress_checked(const df_device_view *v, void *dst, uint32_t *d_err,
                                hipStream_t stream) {
  if (!v || !d_err || !aligned(d_err, 4)) return DF_ERR_ARG;
  void *d[1] = {dst};
  return launch(v, d, 1, d_err, true, stream);
}

df_status df_decompress_batch(const df_device_view *views, void *const *dsts, uint32_t count,
                              hipStream_t stream) {
  return launch(views, dsts, count, nullptr, false, stream);
}

}  // extern "C"
