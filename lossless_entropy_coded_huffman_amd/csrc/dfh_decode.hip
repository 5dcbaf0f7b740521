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
// The gfx950 design:
//   - a tile (the pages' thread block: 256 threads x 8 stream bytes) is
//     decoded by a group of 256 lanes (4 wave64); a workgroup runs up to four
//     such groups, so four tiles share one copy of the tables in LDS (the
//     4096-entry multi-code table, 32 KiB, then the hierarchical tables,
//     512 B each), which lets two 1024-lane workgroups share a CU;
//   - workgroups are persistent and walk the container in steps of
//     (groups x workgroups) tiles, in order; the next step's stream words,
//     gap fields and tile offsets are loaded one step ahead; BF16 keeps that
//     order for three steps, then workgroups take units of four tiles from
//     device-side counters, so faster CUs take more;
//   - a uint8 group takes two neighbouring tiles per step, each lane two
//     neighbouring chunks (its threads 2l and 2l + 1, both with their own
//     gap field): at 6.6-bit codes a chunk holds ten codes, and the step's
//     fixed cost (loads, offsets, scan, barriers) is then spread over
//     twenty;
//   - a BF16 or uint4 group stores a tile one step late.  BF16: the store
//     pass of tile k shares a barrier interval with the count of tile k + 1,
//     so HBM traffic overlaps the decode; the sign|mantissa bytes it merges
//     are requested at the top of the step, before the count.  uint4: the
//     store pass of tile k runs after the scan barrier of tile k + 1, from
//     the other of the group's two staging buffers, so no group barrier
//     ends the step.  A uint8 wave stores its own lanes' output range as
//     soon as its phase 2 is done (plain byte staging needs no clearing, so
//     no group barrier ends the step either);
//   - a lane holds its 8 stream bytes plus the next 4 (uint4: its 16 bytes;
//     uint8: its 16 bytes plus the next 4) in registers and walks each chunk
//     as a 96-bit window shifted with funnel shifts;
//   - a lookup in the multi-code table yields up to five codes (uint8: the
//     pair table, up to two codes from 13 bits); longer codes fall back to
//     the hierarchical tables;
//   - the per-tile prefix sum is a wave64 DPP scan (row_shr, row_bcast) plus
//     one LDS step across the group's four waves;
//   - phase 2 ORs the decoded symbols into the group's LDS staging buffer
//     (uint8: plain byte stores), whose byte j holds output element (tile
//     start rounded down to the store granule) + j, or for uint4 whose
//     nibble j does (the output's own packing, two elements per byte); the
//     store pass reads aligned LDS words, clears them, merges the
//     sign|mantissa bytes (BF16) and issues 16-byte global stores, one in
//     flight per lane (BF16), non-temporal for BF16 and uint4; BF16 also
//     reads its streams non-temporally; the bytes of a partial first or last
//     granule of a uint4 tile or a uint8 range are stored one per lane;
//   - the decode loops run at a raised wave priority, the store pass at the
//     lowest; the uint4 and uint8 kernels replay phase 1's first table
//     entries from registers in phase 2.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>

#include "dfh.h"

namespace {

constexpr uint32_t kTPB = DF_THREADS_PER_TILE;  // lanes per tile group = threads per tile
constexpr uint32_t kMaxGroups = 4;              // tile groups per workgroup
constexpr uint32_t kK = DF_DTAB_BITS;           // multi-code table index width
constexpr uint32_t kDtabEntries = 1u << kK;
constexpr uint32_t kDtabBytes = kDtabEntries * 8;
// uint8: the pair table (13-bit index, two codes per 32-bit entry; 6.6-bit
// codes rarely leave room for a third) and the code length of each symbol
constexpr uint32_t kPairMask = (1u << DF_DTAB_BITS_U8) - 1;
constexpr uint32_t kPairLens = 4u << DF_DTAB_BITS_U8;  // LDS offset of the lengths
// LDS bytes of a kind's decode table (the hierarchical tables follow it)
template <int KIND>
constexpr uint32_t kTabBytes = KIND == DF_KIND_U8 ? (uint32_t)DF_DTAB_BYTES_U8 : kDtabBytes;
constexpr uint32_t kPrefetch = 4;  // sign|mantissa 8-byte groups requested ahead per lane
// s_waitcnt operand (gfx9 encoding: vmcnt in bits 3..0 and 15..14, expcnt
// in 6..4, lgkmcnt in 11..8) that waits for vmcnt 0 only
constexpr int kWaitVm0 = 0x0F70;
// staging positions past a tile's last element that phase 2 may touch: BF16
// and uint8 bytes, up to four lookahead symbol bytes widened to the two words
// of one OR; uint4 nibbles, the two words of one OR (16 nibbles)
template <int KIND>
constexpr uint32_t kSlack = KIND == DF_KIND_U4 ? 16u : 12u;
// Staging buffers per tile group: uint4 two, used by step parity (its steps
// end without a barrier), BF16 and uint8 one.
template <int KIND>
constexpr uint32_t kBufs = KIND == DF_KIND_U4 ? 2u : 1u;
// Table entries phase 1 keeps in registers for phase 2 to replay; a lane
// with more walks the rest of its chunk again from where the kept ones end.
// Counts measured per kind: uint4 keeps 7 (a lane walks about 6 entries at
// 2.7-bit codes; 6 and 8 measured 1.6% and 0.8% slower), uint8 5 of its
// pair-table words per chunk (every unrolled step costs the whole wave, and
// the uint8 kernel is bound by VALU issue; 4 and 6 measured 1.0% and 0.7%
// slower),
// BF16 none (its sign|mantissa prefetch holds the registers: with one or two
// kept entries the kernel spills to scratch).
template <int KIND>
constexpr uint32_t kKeep = KIND == DF_KIND_U4 ? 7u : KIND == DF_KIND_U8 ? 5u : 0u;
template <int KIND>
constexpr uint32_t kKeepRegs = kKeep<KIND> ? kKeep<KIND> : 1u;
// Stream chunks per lane: a uint8 lane walks two neighbouring chunks (a tile
// group decodes two tiles per step).  Measured 11% faster on the uint8
// block; BF16 and uint4 chunks hold 24 codes and keep one.
template <int KIND>
constexpr uint32_t kChunks = KIND == DF_KIND_U8 ? 2u : 1u;

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
  uint32_t ticket;  // the dynamic schedule's first-choice counter slot, or kNoTicket
  uint32_t pad;
};

// Tile counters of the dynamic schedule (BF16).  Each dynamically scheduled
// job of a running dispatch owns one slot of kParts counters on separate
// 128-byte lines (atomics on one address serialize at about 11 ns each on
// MI355X, atomics on separate lines proceed in parallel), plus a line with
// the owner's key and a count of finished counters.  A dispatch claims its
// slot on the device and frees it when its last grab has been served, so no
// state passes from one launch to another and concurrent launches never
// share counters, whatever the host does (graph instances replayed on
// several streams included):
//   - the key is the address of the dispatch's AQL packet (the same for all
//     its workgroups, different for any two dispatches running at once)
//     with the job's index in its six low bits, which a 64-byte packet
//     address leaves zero;
//   - the job's first workgroup claims the first free slot from the host's
//     hint on (compare-and-swap of the owner word from zero to the key),
//     within kWindow slots, waiting for one to free up if all are held;
//   - its other workgroups look for the key in the same slots;
//   - the grab that takes a counter's last value counts that counter as
//     finished; the last counter to finish clears the counters, then frees
//     the slot (a release store of zero to the owner word).
// Every slot is zero when the code object is loaded and zero again when its
// dispatch ends, so no launch clears memory.  All slot accesses are
// system-scope atomics, performed at one coherence point.  A workgroup that
// cannot claim or find its slot within kSpinLimit polls (never seen: it
// would take more than kWindow decodes running at once next to the hint)
// decodes every dynamically dealt unit itself, which covers the job
// whatever its other workgroups do (the writes are identical).
constexpr uint32_t kParts = 8;
constexpr uint32_t kCounterStride = 32;  // u32 words: 128 bytes
constexpr uint32_t kSlotWords = (kParts + 1) * kCounterStride;
constexpr uint32_t kTicketSlots = 4096;
constexpr uint32_t kWindow = 16;
constexpr uint32_t kSpinLimit = 1u << 16;
constexpr uint32_t kNoTicket = 0xFFFFFFFFu;
__device__ uint32_t g_slots[kTicketSlots * kSlotWords];

__device__ __forceinline__ uint64_t *slot_owner(uint32_t s) { return (uint64_t *)(g_slots + (size_t)s * kSlotWords); }
__device__ __forceinline__ uint32_t *slot_done(uint32_t s) { return g_slots + (size_t)s * kSlotWords + 2; }
__device__ __forceinline__ uint32_t *slot_counter(uint32_t s, uint32_t c) {
  return g_slots + (size_t)s * kSlotWords + (c + 1) * kCounterStride;
}
__device__ __forceinline__ uint32_t window_slot(uint32_t hint, uint32_t i) { return (hint + i % kWindow) % kTicketSlots; }

// The first workgroup's claim, given the result of the compare-and-swap it
// made at the hint: the hint, or the first slot of the window it can claim.
__device__ uint32_t claim_slot(uint32_t hint, uint64_t key, uint64_t at_hint) {
  if (at_hint == 0) return hint;
  for (uint32_t k = 1; k < kSpinLimit; k++) {
    if (k % kWindow == 0) __builtin_amdgcn_s_sleep(8);  // every slot held: wait for one
    uint64_t expect = 0;
    if (__hip_atomic_compare_exchange_strong(slot_owner(window_slot(hint, k)), &expect, key, __ATOMIC_RELAXED,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM))
      return window_slot(hint, k);
  }
  return kNoTicket;
}

// Another workgroup's search for the slot its first workgroup claimed: a
// slot held by another key is passed (the claim lies further on); at a free
// slot the claim is awaited, and after a while the search starts over at
// the hint (a slot passed as held may have been freed and then claimed).
__device__ uint32_t find_slot(uint32_t hint, uint64_t key) {
  uint32_t i = 0, waits = 0;
  for (uint32_t k = 0; k < kSpinLimit; k++) {
    const uint32_t s = window_slot(hint, i);
    const uint64_t v = __hip_atomic_load(slot_owner(s), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    if (v == key) return s;
    if (v != 0) {
      i++;
      waits = 0;
      continue;
    }
    __builtin_amdgcn_s_sleep(2);
    if (++waits == 64) i = waits = 0;
  }
  return kNoTicket;
}

// Counter c's last grab of the dispatch has been served.  The last of the
// slot's `parts` counters to finish clears them, then frees the slot.  The
// clears must be done before the owner word reads free: system-scope stores
// are written through to the coherence point and count in vmcnt until it
// acknowledges them, so a vmcnt(0) wait between the two suffices (a release
// store would also write back the whole L2, which the decoder's output
// fills).
__device__ void counter_finished(uint32_t s, uint32_t parts) {
  if (__hip_atomic_fetch_add(slot_done(s), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) + 1 < parts) return;
  for (uint32_t c = 0; c < parts; c++) __hip_atomic_store(slot_counter(s, c), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  __hip_atomic_store(slot_done(s), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __hip_atomic_store(slot_owner(s), (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
// The kinds that use it: with the BF16 block the slowest CUs set the end of a
// static schedule (measured 4.3% faster with it); the uint8 and uint4
// kernels measured 1.5% and 11% slower with it compiled in.
template <int KIND>
constexpr bool kDynamic = KIND == DF_KIND_BF16;

struct Batch {
  Job job[DF_MAX_BATCH];
  uint32_t count;
  uint32_t lut_bytes;  // LDS reserved for hierarchical tables
  uint32_t out_bytes;  // LDS staging bytes per tile group
  uint32_t pad;
  uint32_t *err;       // error word (checked launches only)
};

// LDS is addressed through address-space-3 pointers made from byte offsets:
// the kernel declares no static LDS, so its dynamic LDS starts at offset 0
// and table offsets fold into the ds instructions' immediate fields.
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) v2u lds_v2;
typedef __attribute__((address_space(3))) v4u lds_v4;
// tile offsets are wave-uniform and read through the constant address
// space, which makes them scalar loads
typedef const __attribute__((address_space(4))) uint64_t k_u64;
template <class T>
__device__ __forceinline__ T *lds(uint32_t byte_offset) {
  return (T *)(uintptr_t)byte_offset;
}

// One code through the hierarchical tables (after the kind's decode table):
// returns (length << 8) | symbol.  A prefix with no code (possible only for
// an incomplete code or a corrupt stream) reports DF_DEVERR_CODE in checked
// launches and consumes one bit.
template <int KIND, bool CHECKED>
__device__ __forceinline__ uint32_t long_code(uint32_t n_luts, uint32_t win, uint32_t *err) {
  const lds_u16 *lut = lds<const lds_u16>(kTabBytes<KIND>);
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

// A lane's position in its stream words: b2:b1:b0 holds the stream from
// the current code on (bit 0 of b0 = first bit of the next code).  Built
// from the chunk's three words w2:w1:w0 and the bit g (< 32) at which the
// chunk's first code starts, it keeps every bit a lane reads: codes start
// before chunk bit 64 and are at most 32 bits long.
struct Stream {
  uint32_t b0, b1, b2;
};

__device__ __forceinline__ Stream stream_at(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t g) {
  return {__builtin_amdgcn_alignbit(w1, w0, g), __builtin_amdgcn_alignbit(w2, w1, g), w2 >> g};
}

// Drops the next (s mod 32) bits; s is a table entry's high word, whose
// low five bits are the bits its codes consume (1..12).
__device__ __forceinline__ void drop(Stream &t, uint32_t s) {
  t.b0 = __builtin_amdgcn_alignbit(t.b1, t.b0, s);
  t.b1 = __builtin_amdgcn_alignbit(t.b2, t.b1, s);
  t.b2 = t.b2 >> (s & 31);
}

// Multi-code table entry fields (high word): bits consumed in bits 0..4,
// flags for codes starting at window bits 1..11 in bits 5..15, the fifth
// symbol byte in bits 16..23, the number of codes in bits 24..31; a high
// word below 2^24 marks a first code longer than the table's index width.
constexpr uint32_t kOneCode = 1u << 24;

// ORs an entry's symbol bytes (low word: codes 0..3, high word bits 16..23:
// code 4) into the staging buffer at byte q.
__device__ __forceinline__ void or_entry(uint32_t q, v2u e) {
  const uint64_t v = ((((uint64_t)((e.y >> 16) & 0xFFu)) << 32) | e.x) << ((q & 3) * 8);
  lds_u32 *w = lds<lds_u32>(q & ~3u);
  __hip_atomic_fetch_or(w, (uint32_t)v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  __hip_atomic_fetch_or(w + 1, (uint32_t)(v >> 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// uint4: ORs an entry's symbols (nibbles, low word bits 0..19) into the
// staging buffer at nibble q (nibble 2j + i of the buffer is the low (i = 0)
// or high nibble of byte j, the output's own packing).  Against byte staging
// packed into nibbles by the store pass, the uint4 block went from 76.7 to
// 71.0 us side by side: the store pass copies granules, and reads and
// clears half the LDS bytes.
__device__ __forceinline__ void or_nibbles(uint32_t q, uint32_t x) {
  const uint64_t v = (uint64_t)x << ((q & 7) * 4);
  lds_u32 *w = lds<lds_u32>((q >> 3) << 2);
  __hip_atomic_fetch_or(w, (uint32_t)v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  __hip_atomic_fetch_or(w + 1, (uint32_t)(v >> 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Stores a pair-table entry's symbol bytes (bits 8..23) at staging byte q:
// the first always, the second when the entry holds two codes.  uint8 lanes
// store plain bytes rather than OR words: every byte a lane stores is either
// its own or the same value the lane that owns it stores (a walk's last
// entry reaches into the next chunk's first codes), and an entry of no codes
// (a kept run parked at a long code) stores a zero that the lane's own walk
// overwrites later; so the staging buffer needs no clearing between tiles.
// Measured 3.7% faster on the uint8 block than two LDS ORs per entry.
__device__ __forceinline__ void put_pair(uint32_t q, uint32_t h) {
  lds_u8 *p = lds<lds_u8>(q);
  p[0] = (uint8_t)(h >> 8);
  if (h >= 2u << 24) p[1] = (uint8_t)(h >> 16);
}

// In place of a table entry whose first code is longer than the index width:
// an entry for that one code (symbol byte in the low word for phase 2).  A
// 32-bit code, whose length does not fit the five-bit field, drops one
// stream word here and reports 0 bits (phase 1 takes the 32 bits off its
// budget itself).
template <int KIND, bool CHECKED>
__device__ __forceinline__ v2u long_entry(uint32_t n_luts, Stream &t, uint32_t *err) {
  const uint32_t c = long_code<KIND, CHECKED>(n_luts, t.b0, err);
  uint32_t len = c >> 8;
  if (len >= 32) {
    t.b0 = t.b1;
    t.b1 = t.b2;
    t.b2 = 0;
    len = 0;
  }
  const uint32_t sym = KIND == DF_KIND_BF16 ? rot_right1(c & 0xFFu) : KIND == DF_KIND_U4 ? (c & 0xFu) : (c & 0xFFu);
  if (KIND == DF_KIND_U8) return (v2u){0u, kOneCode | (sym << 8) | len};  // a pair-table entry
  return (v2u){sym, kOneCode | len};
}

// The streams that are read once (stream words, sign|mantissa bytes) are
// loaded, and the BF16 output stored, non-temporally: with all three the
// BF16 block ran 1% faster (139.4 against 140.7 us, on three boxes); the
// loads or the stores alone were neutral or up to 2% slower, and the uint8
// and uint4 kernels measured the same either way.
__device__ __forceinline__ uint2 load_nt2(const void *p) {
  const v2u v = __builtin_nontemporal_load((const v2u *)p);
  return make_uint2(v.x, v.y);
}

// BF16 element stores of the part of a 16-byte store granule that lies in
// [lo, hi) (granules shared with a neighbouring tile).  (Spreading these
// elements over lanes, their sign|mantissa bytes read from the granule's
// lane, made the BF16 block 29% slower; every wave then read the last
// granule lane's prefetch register before its loop, so it waited for its
// prefetched loads at once rather than one granule at a time.  Handing the
// merged granule to eight lanes of the owner's wave through LDS instead
// measured the same as these stores: BF16 is bound by its memory path.)
__device__ __forceinline__ void store_partial(uint16_t *dst, uint32_t e0, uint32_t lo, uint32_t hi, uint4 o) {
#pragma unroll
  for (uint32_t i = 0; i < 8; i++) {
    const uint32_t w = i < 2 ? o.x : i < 4 ? o.y : i < 6 ? o.z : o.w;
    if (e0 + i >= lo && e0 + i < hi) dst[e0 + i] = (uint16_t)(w >> (16 * (i & 1)));
  }
}

// The store pass of one tile (BF16 and uint4; uint8 waves store their own
// ranges in the step loop): aligned 16-byte stores of output elements
// [a + lo_r, a + hi_r) from the staging buffer at LDS byte buf; BF16 merges
// each granule's exponents with its sign|mantissa bytes (the first
// kPrefetch granules of each lane arrive in smv, the rest are loaded here).
// A BF16 lane keeps one store in flight: it waits for the previous store
// (s_waitcnt vmcnt(0), which also covers the next step's stream words,
// requested before the count and back by then) before the next.  When
// every wave issued its stores back to back, the write bursts delayed the
// stream and sign|mantissa loads that the decode waits on, and the kernel
// ran about 5% slower.
//
// The pass also leaves the staging buffer zero for the next tile's ORs:
// each lane clears the granules it has just read, and the bytes from the
// last granule up to `dirty` (the next lane-group's lookahead slack) are
// cleared here too.
//
// uint4 staging holds nibbles in the output's packing, so a granule of 32
// elements is 16 staging bytes copied as they are; a tile owns the output
// bytes whose low-nibble element is its own, [ceil(lo / 2), ceil(hi / 2))
// relative to a / 2; he is hi_r + 1 when the element after the tile exists
// (its symbol then sits at staging nibble hi_r), else hi_r.
template <int KIND>
__device__ __forceinline__ void store_tile(const Job &jb, uint32_t buf, uint64_t a, uint32_t lo_r,
                                           uint32_t hi_r, uint32_t he, uint32_t ngroups, uint32_t dirty,
                                           const uint2 (&smv)[kPrefetch], uint32_t lane) {
  static_assert(KIND != DF_KIND_U8, "uint8 waves store their own ranges");
  const uint32_t gbytes = 16u / (KIND == DF_KIND_BF16 ? 2u : 1u);  // staging bytes per store granule
  for (uint32_t o = gbytes * ngroups + 8 * lane; o < dirty; o += 8 * kTPB)
    *lds<lds_v2>(buf + o) = (v2u){0u, 0u};
  if (KIND == DF_KIND_BF16) {
    uint16_t *dst_t = (uint16_t *)jb.dst + a;
    const uint8_t *sm_t = jb.sm + a;
    lds_v2 *ex_t = lds<lds_v2>(buf);
#pragma unroll
    for (uint32_t k = 0; k < kPrefetch; k++) {
      const uint32_t g = lane + k * kTPB;
      if (k > 0) __builtin_amdgcn_s_waitcnt(kWaitVm0);
      if (g < ngroups) {
        const uint32_t e0 = 8 * g;
        const v2u ex = ex_t[g];
        ex_t[g] = (v2u){0u, 0u};
        const uint2 o01 = merge4(ex.x, smv[k].x);
        const uint2 o23 = merge4(ex.y, smv[k].y);
        const uint4 o = make_uint4(o01.x, o01.y, o23.x, o23.y);
        if (e0 >= lo_r && e0 + 8 <= hi_r) __builtin_nontemporal_store((v4u){o.x, o.y, o.z, o.w}, (v4u *)(dst_t + e0));
        else store_partial(dst_t, e0, lo_r, hi_r, o);
      }
    }
    for (uint32_t g = lane + kPrefetch * kTPB; g < ngroups; g += kTPB) {
      const uint32_t e0 = 8 * g;
      const v2u ex = ex_t[g];
      ex_t[g] = (v2u){0u, 0u};
      // a plain load: this loop runs only for tiles of more than 8192
      // elements, and with a non-temporal load here the compiler kept 64-bit
      // addresses that spilled a register to scratch
      const uint2 sv = *(const uint2 *)(sm_t + e0);
      const uint2 o01 = merge4(ex.x, sv.x);
      const uint2 o23 = merge4(ex.y, sv.y);
      const uint4 o = make_uint4(o01.x, o01.y, o23.x, o23.y);
      if (e0 >= lo_r && e0 + 8 <= hi_r) __builtin_nontemporal_store((v4u){o.x, o.y, o.z, o.w}, (v4u *)(dst_t + e0));
      else store_partial(dst_t, e0, lo_r, hi_r, o);
    }
  } else if (KIND == DF_KIND_U4) {
    uint8_t *dst_t = (uint8_t *)jb.dst + a / 2;
    lds_v4 *ex_t = lds<lds_v4>(buf);
    const uint32_t blo = (lo_r + 1) / 2, bhi = (hi_r + 1) / 2;
    // the last byte's high nibble when no element follows the tile
    const uint32_t kill = (he == hi_r && (hi_r & 1)) ? bhi - 1 : 0xFFFFFFFFu;
    // whole granules [fs, fe) in the loop, then the bytes of a partial
    // first or last granule one per lane (lanes 0..15 the first, 16..31 the
    // last): one predicated byte store for the wave, where a 16-step byte
    // loop in one lane held its whole wave (the uint4 block went from 85.2
    // to 77.2 us side by side)
    const uint32_t fs = (blo + 15) / 16, fe = bhi / 16;
    for (uint32_t g = fs + lane; g < fe; g += kTPB) {
      v4u o = ex_t[g];
      ex_t[g] = (v4u){0u, 0u, 0u, 0u};
      const uint32_t b0 = 16 * g;
      if (kill - b0 < 16) {
        const uint32_t m = ~(0xF0u << (8 * ((kill - b0) & 3)));
        const uint32_t wk = (kill - b0) >> 2;
        o.x &= wk == 0 ? m : ~0u;
        o.y &= wk == 1 ? m : ~0u;
        o.z &= wk == 2 ? m : ~0u;
        o.w &= wk == 3 ? m : ~0u;
      }
      // non-temporal: 2.4% faster on the uint4 block (uint8 the same)
      __builtin_nontemporal_store(o, (v4u *)(dst_t + b0));
    }
    // (granules 0 and ngroups - 1 are the only ones outside [fs, fe), as
    // blo <= 16 and 16 (ngroups - 1) < bhi; each is read and cleared whole,
    // its 16 staging bytes, also where the tile owns none of its output
    // bytes)
    if (lane < 32 && ngroups > 0) {
      const uint32_t g = lane < 16 ? 0u : ngroups - 1;
      const uint32_t p = 16 * g + (lane & 15);
      if (g < fs || g >= fe) {
        lds_u8 *sb = lds<lds_u8>(buf + p);
        uint32_t byte = *sb;
        *sb = 0;
        if (p == kill) byte &= 0x0Fu;
        if (p >= blo && p < bhi) dst_t[p] = (uint8_t)byte;
      }
    }
  }
}

struct ChunkRegs {
  // w3: uint4 (next-tile code, below) and uint8 (second chunk); w4: uint8
  uint32_t w0, w1, w2, w3, w4, g0, g1;
};

// The stream words and gap fields of one lane of a span (kChunks tiles).
// Addresses are a wave-uniform base plus a 32-bit lane offset.
// A span past the last (a group with no next span) reads the last span
// again: the loads are issued on every path, so each step puts the same
// number of loads in flight, in the same order.  In a last span of one tile
// (uint8, odd tile count) the lanes of the missing tile read lane 0's words.
// Reads stay inside the sections: a lane's lookahead word and its second
// gap word lie at most four bytes past its tile's end, inside the 16 bytes
// of padding.  Needs n_tiles >= 1.
template <int KIND>
__device__ __forceinline__ ChunkRegs load_chunk(const Job &jb, uint32_t span, uint32_t lane) {
  constexpr uint32_t C = kChunks<KIND>;
  const uint32_t n_spans = ((uint32_t)jb.n_tiles + C - 1) / C;
  if (span >= n_spans) span = n_spans - 1;
  if (C > 1 && C * span + (C * lane) / kTPB >= (uint32_t)jb.n_tiles) lane = 0;
  ChunkRegs c;
  const uint32_t *bits_t = jb.bits + (uint64_t)span * (2 * C * kTPB);
  const uint2 w01 = load_nt2(bits_t + 2 * C * lane);
  c.w0 = w01.x;
  c.w1 = w01.y;
  c.w4 = 0;
  if (KIND == DF_KIND_U4 || C == 2) {  // 128 bits (the stream has 16 bytes of padding)
    const uint2 w23 = *(const uint2 *)(bits_t + 2 * C * lane + 2);
    c.w2 = w23.x;
    c.w3 = w23.y;
    if (C == 2) c.w4 = bits_t[4 * lane + 4];
  } else {
    c.w2 = bits_t[2 * lane + 2];
    c.w3 = 0;
  }
  const uint32_t *gaps_t = jb.gaps + (uint64_t)span * (5 * C * kTPB / 32);  // 1280 bits per tile
  c.g0 = gaps_t[(5 * C * lane) >> 5];
  c.g1 = gaps_t[((5 * C * lane) >> 5) + 1];
  return c;
}

// Phase 1 over one chunk: counts the codes that start in [gap, E), walking
// from t (the stream at gap) with rem = E - gap bits before E.  Whole
// entries are counted; the entry that crosses E gives back its codes that
// start at or past E (they are the next chunk's first codes).  The walk's
// first kKeep entries go to registers for phase 2 (symbol words, and the
// high halves of the high words two to a register) and t is left past them;
// rem_end is E minus where the walk stopped (<= 0).
template <int KIND, bool CHECKED>
__device__ __forceinline__ uint32_t count_chunk(Stream &t, int32_t rem, uint32_t (&kept_lo)[kKeepRegs<KIND>],
                                                uint32_t (&kept_hi)[(kKeepRegs<KIND> + 1) / 2],
                                                int32_t &rem_end, uint32_t n_luts, uint32_t *err) {
  uint32_t cnt = 0, h = 0;
  if (KIND == DF_KIND_U8) {
    // A lane past E takes an entry of no codes, and so does a lane at a
    // code longer than the table's index width (staging leaves such table
    // entries zero): its window stays put, so each later kept entry is
    // empty too, and the loop below resumes the walk there.  This
    // branch-free form measured 3% faster on the uint8 block than the
    // guarded one below.  The bits consumed are the entry's low byte (bits
    // 4..7 are zero: staging clears them).  h is left at a zero entry only
    // for a lane parked at a long code, whose loop below runs and sets it.
#pragma unroll
    for (uint32_t k = 0; k < kKeep<KIND>; k++) {
      const bool live = rem > 0;
      uint32_t y = lds<const lds_u32>(0)[t.b0 & kPairMask];
      if (!live) y = 0;
      drop(t, y);
      rem -= (int32_t)(y & 0xFFu);
      cnt += y >> 24;
      if (live) h = y;
      kept_lo[k] = y;
    }
  } else {
    // At the lane's first code longer than the table's index width the
    // table entry is zero (staging leaves it so): the window stays put and
    // each later kept entry is the same empty one, and the loop below
    // resumes the walk there.  Without a separate flag for that case the
    // uint4 block went from 71.4 to 65.2 us.  (The branch-free form, every
    // kept lookup in every lane, measured 68.3 against 65.1 us: a lane past
    // the chunk end skips its remaining lookups here, and their LDS reads.)
#pragma unroll
    for (uint32_t k = 0; k < kKeep<KIND>; k++) {
      v2u e = {0u, 0u};
      if (rem > 0) {
        e = lds<const lds_v2>(0)[t.b0 & (kDtabEntries - 1)];
        drop(t, e.y);
        rem -= (int32_t)(e.y & 31);
        cnt += e.y >> 24;
        h = e.y;
      }
      kept_lo[k] = e.x;
      if (k & 1) kept_hi[k / 2] |= e.y & 0xFFFF0000u;
      else kept_hi[k / 2] = e.y >> 16;
    }
  }
  Stream t2 = t;
  while (rem > 0) {
    h = KIND == DF_KIND_U8 ? lds<const lds_u32>(0)[t2.b0 & kPairMask]
                           : lds<const lds_u32>(4)[(t2.b0 & (kDtabEntries - 1)) << 1];
    if (h < kOneCode) {  // rare: a code longer than the table's index width
      h = long_entry<KIND, CHECKED>(n_luts, t2, err).y;
      if ((h & 31) == 0) rem -= 32;
    }
    drop(t2, h);
    rem -= (int32_t)(h & (KIND == DF_KIND_U8 ? 0xFFu : 31u));
    cnt += h >> 24;
  }
  if (rem < 0) {
    // bits of the last entry before E (1..12; a one-code entry has no flags)
    const uint32_t r = (uint32_t)(rem + (int32_t)(h & 31));
    if (KIND == DF_KIND_U8) {
      // a pair: the second code starts at (consumed - its length)
      if ((h >> 24) == 2 && (h & 31) - lds<const lds_u8>(kPairLens)[(h >> 16) & 0xFFu] >= r) cnt -= 1;
    } else {
      cnt -= (h >> 24) - 1 - __popc(__builtin_amdgcn_ubfe(h, 5, (r - 1) & 15));
    }
  }
  rem_end = rem;
  return cnt;
}

// Phase 2 over one chunk: the same entries again (those phase 1 kept are
// replayed from registers, the rest decoded again from t), their symbol
// bytes ORed into the staging buffer from byte q until qend.  Returns where
// the writes stopped (the last entry's codes past qend included).
template <int KIND, bool CHECKED>
__device__ __forceinline__ uint32_t write_chunk(uint32_t q, uint32_t qend, Stream t,
                                                const uint32_t (&kept_lo)[kKeepRegs<KIND>],
                                                const uint32_t (&kept_hi)[(kKeepRegs<KIND> + 1) / 2],
                                                uint32_t n_luts, uint32_t *err) {
#pragma unroll
  for (uint32_t k = 0; k < kKeep<KIND>; k++)
    if (q < qend) {
      if (KIND == DF_KIND_U8) {
        put_pair(q, kept_lo[k]);
        q += kept_lo[k] >> 24;
      } else {  // (uint4: BF16 keeps none)
        const uint32_t hi = (k & 1) ? kept_hi[k / 2] & 0xFFFF0000u : kept_hi[k / 2] << 16;
        or_nibbles(q, kept_lo[k]);
        q += hi >> 24;
      }
    }
  if (KIND == DF_KIND_U8) {
    while (q < qend) {
      uint32_t h = lds<const lds_u32>(0)[t.b0 & kPairMask];
      if (h < kOneCode) h = long_entry<KIND, CHECKED>(n_luts, t, err).y;  // rare
      drop(t, h);
      put_pair(q, h);
      q += h >> 24;
    }
  } else {
    while (q < qend) {
      v2u e = lds<const lds_v2>(0)[t.b0 & (kDtabEntries - 1)];
      if (e.y < kOneCode) e = long_entry<KIND, CHECKED>(n_luts, t, err);  // rare
      drop(t, e.y);
      if (KIND == DF_KIND_U4) or_nibbles(q, e.x);
      else or_entry(q, e);
      q += e.y >> 24;
    }
  }
  return q;
}

// A decode-table word (16 bytes) on its way to LDS: an entry that claims
// codes but consumes no bits would never move a walk forward, so it is
// cleared (a cleared entry sends the walk to the hierarchical tables, which
// consume at least one bit per code) and, in checked launches, reported as
// DF_DEVERR_CODE.  Tables built by the library never hold such entries; a
// caller-made view with a damaged table pointer may.  An entry that claims
// no codes (a window whose first code is longer than the index width) is
// cleared whole (the library's are zero already), so the kept runs of
// phase 1 can take it as is: it moves nothing and counts nothing.  Entries: BF16 and
// uint4 two u64 (high words y and w), uint8 four u32 pair entries (the
// lengths that follow the pair table are left alone), whose bits 5..7 are
// cleared as well: phase 1 reads an entry's bits consumed as its low byte,
// and they must match what a walk drops (the low five bits).
template <int KIND, bool CHECKED>
__device__ __forceinline__ v4u clean_tab(v4u v, uint32_t word, uint32_t *err) {
  bool bad = false;
  if (KIND == DF_KIND_U8) {
    if (word < (4u << DF_DTAB_BITS_U8) / 16) {
#pragma unroll
      for (int c = 0; c < 4; c++) {
        if (v[c] >= kOneCode && (v[c] & 31u) == 0) {
          v[c] = 0;
          bad = true;
        }
        if (v[c] < kOneCode) v[c] = 0;
        v[c] &= ~0xE0u;
      }
    }
  } else {
    if (v.y >= kOneCode && (v.y & 31u) == 0) {
      v.x = v.y = 0;
      bad = true;
    }
    if (v.w >= kOneCode && (v.w & 31u) == 0) {
      v.z = v.w = 0;
      bad = true;
    }
    if (v.y < kOneCode) v.x = v.y = 0;
    if (v.w < kOneCode) v.z = v.w = 0;
  }
  if (CHECKED && bad) atomicOr(err, DF_DEVERR_CODE);
  return v;
}

// PRIO: the decode loops run at a raised wave priority (the default); a
// launch with a workgroup cap, which shares the CUs with kernels running
// beside it, uses PRIO = false and stays at the base priority.  (A runtime
// flag instead of a template parameter cost the BF16 kernel registers and
// 1.2% of its time.)
template <int KIND, bool CHECKED, bool PRIO>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(8)))
void decode_kernel(const Batch batch) {
  // LDS (all dynamic, from offset 0): the decode table, hierarchical tables,
  // the staging buffers of each tile group (uint4 two), two sets of
  // per-wave scan sums (32 bytes per group; uint8 and uint4 alternate between
  // them), then 64 bytes for the dynamic schedule
  const uint32_t wg = blockIdx.x;
  uint32_t j = 0;
  while (j + 1 < batch.count && wg >= batch.job[j + 1].wg_begin) j++;
  const Job &jb = batch.job[j];
  const uint32_t tid = threadIdx.x;
  const uint32_t groups = blockDim.x / kTPB;
  const uint32_t grp = __builtin_amdgcn_readfirstlane(tid / kTPB);
  const uint32_t lane = tid % kTPB;
  const uint32_t n_luts = jb.n_luts;
  const uint32_t out_bytes = batch.out_bytes;
  const uint32_t buf0 = kTabBytes<KIND> + batch.lut_bytes + grp * kBufs<KIND> * out_bytes;  // LDS byte offset
  lds_u32 *wsum = lds<lds_u32>(kTabBytes<KIND> + batch.lut_bytes + groups * kBufs<KIND> * out_bytes);

  // dynamic schedule (BF16): the job's first workgroup claims a counter
  // slot, the others look for its key (requested behind the table loads
  // below, read after the staging)
  const bool dyn = kDynamic<KIND> && jb.ticket != kNoTicket;
  const bool lead = wg == jb.wg_begin;
  const uint64_t key = (uint64_t)(uintptr_t)__builtin_amdgcn_dispatch_ptr() | (j + 1);
  uint64_t at_hint = 0;
  {  // stage the tables once per workgroup: the first four 16-byte words per
     // lane (all a 1024-lane workgroup needs for up to 64 levels) with every
     // load issued before any write, the rest one by one
    constexpr uint32_t kTabWords = kTabBytes<KIND> / 16;
    const uint32_t total = kTabWords + n_luts * 32;  // 16-byte words: table, then levels
    const v4u *dsrc = (const v4u *)jb.dtab;
    const v4u *lsrc = (const v4u *)jb.lut - kTabWords;
    lds_v4 *dl = lds<lds_v4>(0);
    const uint32_t i0 = tid, i1 = tid + blockDim.x, i2 = tid + 2 * blockDim.x, i3 = tid + 3 * blockDim.x;
    const v4u z = {0u, 0u, 0u, 0u};
    const v4u t0 = i0 < total ? (i0 < kTabWords ? dsrc[i0] : lsrc[i0]) : z;
    const v4u t1 = i1 < total ? (i1 < kTabWords ? dsrc[i1] : lsrc[i1]) : z;
    const v4u t2 = i2 < total ? (i2 < kTabWords ? dsrc[i2] : lsrc[i2]) : z;
    const v4u t3 = i3 < total ? (i3 < kTabWords ? dsrc[i3] : lsrc[i3]) : z;
    if (dyn && tid == 0) {
      if (lead) {
        uint64_t expect = 0;
        __hip_atomic_compare_exchange_strong(slot_owner(jb.ticket), &expect, key, __ATOMIC_RELAXED,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        at_hint = expect;
      } else {
        at_hint = __hip_atomic_load(slot_owner(jb.ticket), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      }
    }
    if (i0 < total) dl[i0] = i0 < kTabWords ? clean_tab<KIND, CHECKED>(t0, i0, batch.err) : t0;
    if (i1 < total) dl[i1] = i1 < kTabWords ? clean_tab<KIND, CHECKED>(t1, i1, batch.err) : t1;
    if (i2 < total) dl[i2] = i2 < kTabWords ? clean_tab<KIND, CHECKED>(t2, i2, batch.err) : t2;
    if (i3 < total) dl[i3] = i3 < kTabWords ? clean_tab<KIND, CHECKED>(t3, i3, batch.err) : t3;
    for (uint32_t i = tid + 4 * blockDim.x; i < total; i += blockDim.x)
      dl[i] = i < kTabWords ? clean_tab<KIND, CHECKED>(dsrc[i], i, batch.err) : lsrc[i];
  }

  // Tile schedule, in spans of kChunks tiles (one tile but for uint8).
  // Static: the job's G = groups x workgroups tile groups take spans in
  // order, workgroup w's first span at step k being k G + w groups (base).
  // Dynamic (kDynamic, a counter slot given, more than 3G tiles): the
  // first three steps the same; after that the units of
  // `groups` tiles from 3G on are dealt by kParts counters in turn (unit
  // 3 W + P j + c from grab j of counter c, W workgroups, P counters), and a
  // workgroup grabs its next unit from counter c = (w / 8) mod P, so every
  // counter serves workgroups on every XCD.  A grab is made in step k after
  // the scan barrier, once the workgroup knows it has tiles in step k + 2;
  // it is read in step k + 1, for step k + 3: its latency lies under phase 2
  // and the next count.  Every workgroup ends with one grab that gives no
  // tile, so counter c is grabbed V + W_c times (V grabs with tiles, W_c
  // workgroups); the grab that returns V + W_c - 1 is its last use and
  // stores zero.  Workgroups on faster CUs take more tiles.
  constexpr uint32_t C = kChunks<KIND>;
  // tile and span indices are 32-bit (the host takes fewer than 2^31 tiles)
  const uint32_t n_tiles = (uint32_t)jb.n_tiles;
  const uint32_t n_spans = (n_tiles + C - 1) / C;
  const uint32_t step = jb.wg_count * groups;
  uint32_t base = (wg - jb.wg_begin) * groups;
  uint32_t base_nxt = base + step;  // the workgroup's first tile next step
  // the one lane that grabs (thread 0) keeps the schedule's state in LDS:
  // word 0 the published first tile (0xFFFFFFFF: none), 1 the slot
  // (kNoTicket: not known yet), 2..3 the counter's address (0: the
  // workgroup deals units to itself, no slot found), 4 the first unit, 5 the
  // unit stride, 6 the counter's last value, 7 the counter c, plus 16 once
  // its last value has been taken, plus 32 when the workgroup deals units to
  // itself, 8..9 the key, 10 the number of counters
  lds_u32 *nx_lds = lds<lds_u32>(kTabBytes<KIND> + batch.lut_bytes + groups * kBufs<KIND> * out_bytes + 32 * groups);
  if (dyn && tid == 0) {
    const uint32_t nwg = jb.wg_count, w = wg - jb.wg_begin;
    const uint32_t parts = nwg / 8 < kParts ? (nwg / 8 ? nwg / 8 : 1u) : kParts;
    const uint32_t c = (w >> 3) % parts;
    const uint32_t oct = nwg >> 3, odd = nwg & 7;  // workgroups of counter c
    const uint32_t wc = 8 * (oct / parts + (c < oct % parts ? 1u : 0u)) + (odd && oct % parts == c ? odd : 0u);
    const uint32_t units = (n_spans + groups - 1) / groups;
    const uint32_t first = 3 * nwg + c;
    const uint32_t vc = units > first ? (units - first + parts - 1) / parts : 0u;
    // the lead's claim is settled here; another workgroup that did not see
    // its key at the hint yet searches at its first grab
    const uint32_t sl = lead ? claim_slot(jb.ticket, key, at_hint) : at_hint == key ? jb.ticket : kNoTicket;
    nx_lds[1] = sl;
    nx_lds[4] = first;
    nx_lds[5] = parts;
    nx_lds[6] = (uint32_t)(vc + wc - 1);
    nx_lds[7] = c;
    nx_lds[8] = (uint32_t)key;
    nx_lds[9] = (uint32_t)(key >> 32);
    nx_lds[10] = parts;
    const uint64_t cp = sl == kNoTicket ? 0 : (uint64_t)(uintptr_t)slot_counter(sl, c);
    nx_lds[2] = (uint32_t)cp;
    nx_lds[3] = (uint32_t)(cp >> 32);
    if (lead && sl == kNoTicket) {  // no slot: deal every unit to itself
      nx_lds[4] = 3 * nwg;
      nx_lds[5] = 1;
      nx_lds[6] = 0xFFFFFFFFu;
      nx_lds[7] = 32;
    }
  }
  bool first_step = true, grabbed = false;
  // the grab in flight (lane 0 of the workgroup); a workgroup that deals
  // units to itself counts its grabs here, so the first gives unit 0
  uint32_t tk = 0xFFFFFFFFu;
  ChunkRegs nxt = load_chunk<KIND>(jb, base + grp, lane);
  // the next span's first and last output index, one step ahead
  k_u64 *tout = (k_u64 *)jb.tile_out;
  uint64_t nlo = 0, nhi = 0;
  if (base + grp < n_spans) {
    nlo = tout[C * (base + grp)];
    nhi = tout[C * (base + grp) + C < n_tiles ? C * (base + grp) + C : n_tiles];
  }
  {  // the staging buffer starts zero (out_bytes is a multiple of 16)
    lds_v4 *z = lds<lds_v4>(buf0);
    for (uint32_t i = lane; i < kBufs<KIND> * out_bytes / 16; i += kTPB) z[i] = (v4u){0u, 0u, 0u, 0u};
  }
  __syncthreads();

  // The previous tile of this group is stored one step late.  BF16: while
  // this step counts, so the store pass (HBM-heavy) shares a barrier
  // interval with phase 1 (LDS- and ALU-heavy); it reads the staging buffer
  // before phase 2 writes it again (a barrier lies between) and clears what
  // it reads, so one buffer per group suffices.  uint4: right after the scan
  // barrier, from the other of its two buffers, which phase 2 writes again
  // only after the next scan barrier; so the step needs no barrier at its
  // end (uint4 block 65.0 -> 61.3 us side by side; the store after phase 2
  // instead, 63.7 us).
  bool have_prev = false;
  uint64_t prev_a = 0;
  uint32_t prev_lo = 0, prev_hi = 0, prev_he = 0, prev_ng = 0, prev_dirty = 0;

  uint32_t par = 0;  // step parity
  for (; base < n_spans;) {
    const uint32_t tile = base + grp;  // the span, wave-uniform
    const uint32_t buf = buf0 + (kBufs<KIND> == 2 ? par * out_bytes : 0u);  // this step's staging
    const uint32_t pbuf = buf0 + (kBufs<KIND> == 2 ? (par ^ 1u) * out_bytes : 0u);  // the previous step's
    const bool active = tile < n_spans;
    // The previous tile's first sign|mantissa granules go in flight first
    // (granules past the tile read its last one; step 0 reads granule 0),
    // then the wait for this step's stream words leaves exactly these loads
    // outstanding (the memory counter retires in order), then the next
    // step's words go in flight.
    uint2 smv[kPrefetch];
    if (KIND == DF_KIND_BF16) {
      // a uniform base and 32-bit lane offsets
      const uint8_t *sm_a = jb.sm + prev_a;
      const uint32_t last = prev_ng ? prev_ng - 1 : 0u;
#pragma unroll
      for (uint32_t k = 0; k < kPrefetch; k++) {
        const uint32_t g = lane + k * kTPB;
        smv[k] = load_nt2(sm_a + 8 * (g < prev_ng ? g : last));
      }
    }
    const ChunkRegs cur = nxt;
    asm volatile("" ::"v"(cur.w0), "v"(cur.w1), "v"(cur.w2), "v"(cur.g0), "v"(cur.g1));
    if (KIND == DF_KIND_U4) asm volatile("" ::"v"(cur.w3));
    uint64_t lo = nlo, hi = nhi;
    const uint32_t next = (kDynamic<KIND> ? base_nxt : base + step) + grp;  // next step's tile
    nxt = load_chunk<KIND>(jb, next, lane);
    if (next < n_spans) {
      nlo = tout[C * next];
      nhi = tout[C * next + C < n_tiles ? C * next + C : n_tiles];
    }
    if (hi > jb.n) hi = jb.n;
    if (lo > hi) lo = hi;
    if (hi - lo > C * jb.max_tile_elems) hi = lo + C * jb.max_tile_elems;
    // output range relative to the store-granule-aligned base a
    const uint64_t a = KIND == DF_KIND_BF16 ? (lo & ~7ull) : KIND == DF_KIND_U8 ? (lo & ~15ull) : (lo & ~31ull);
    const uint32_t lo_r = (uint32_t)(lo - a), hi_r = (uint32_t)(hi - a);
    // elements per 16-byte store granule
    const uint32_t gsz = KIND == DF_KIND_BF16 ? 8u : KIND == DF_KIND_U8 ? 16u : 32u;
    const uint32_t ngroups = active ? (hi_r + gsz - 1) / gsz : 0u;

    // chunk bounds: codes start in [gap, E) of this lane's (first) 64
    // stream bits, and in [gap2, E2) of its second chunk (uint8)
    uint32_t gap = 0, E = 0, gap2 = 0, E2 = 0;
    const uint64_t bits_left = jb.total_bits - (uint64_t)tile * (64 * C * kTPB);  // uniform
    if (KIND != DF_KIND_BF16 && active && __builtin_expect(bits_left >= 64 * (uint64_t)(C * kTPB), 1)) {
      // a whole span (all but a container's last): every lane has all its
      // chunks, 64 bits each, so no lane needs the per-lane bounds below
      // (uint8 and uint4 -1.3% and -1.6%; BF16 measured 0.4% slower with it)
      const uint32_t f = (uint32_t)(((((uint64_t)cur.g1) << 32) | cur.g0) >> ((5 * C * lane) & 31));
      gap = f & 31u;
      E = 64;
      if (C == 2) {
        gap2 = (f >> 5) & 31u;
        E2 = 64;
      }
    } else if (active) {
      const uint64_t chunks_left = jb.n_threads - (uint64_t)tile * (C * kTPB);  // > 0 for an active span
      if (C * lane < chunks_left) {
        const uint32_t f = (uint32_t)(((((uint64_t)cur.g1) << 32) | cur.g0) >> ((5 * C * lane) & 31));
        gap = f & 31u;
        if (bits_left >= 64 * (uint64_t)(C * kTPB)) {
          E = 64;
          E2 = C == 2 ? 64u : 0u;
        } else {
          const uint32_t r = (uint32_t)bits_left - 64 * C * lane;
          E = r < 64 ? r : 64u;
          if (C == 2) E2 = r < 64 ? 0u : r - 64 < 64 ? r - 64 : 64u;
        }
        if (C == 2 && C * lane + 1 < chunks_left) gap2 = (f >> 5) & 31u;
        else E2 = 0;
      }
    }

    // The decode loops (dependent lookup chains) run at a raised wave
    // priority, the store pass and the scan at the lowest: when waves of a
    // SIMD compete for issue, the chains go first and the stores fill in
    // (measured: about 1% on the BF16 block, 3% on uint8).  A capped launch
    // (PRIO = false), which shares the CUs with kernels running beside it,
    // stays at the base priority so that it does not take issue slots ahead
    // of them.
    if (PRIO) __builtin_amdgcn_s_setprio(3);
    // phase 1: count the codes that start in the lane's chunks
    int32_t rem_end = 0;  // E minus where the first chunk's walk stopped (<= 0)
    uint32_t kept_lo[kKeepRegs<KIND>], kept_hi[(kKeepRegs<KIND> + 1) / 2];
    Stream after = stream_at(cur.w0, cur.w1, cur.w2, gap);  // the walk past the kept entries
    uint32_t cnt = count_chunk<KIND, CHECKED>(after, (int32_t)(E - gap), kept_lo, kept_hi, rem_end, n_luts,
                                             batch.err);
    // the second chunk (uint8): words w2..w4, codes from 64 + gap2
    uint32_t cnt1 = cnt;
    uint32_t kept2_lo[kKeepRegs<KIND>], kept2_hi[(kKeepRegs<KIND> + 1) / 2];
    Stream after2 = {0u, 0u, 0u};
    if constexpr (C == 2) {
      int32_t rem_end2 = 0;
      after2 = stream_at(cur.w2, cur.w3, cur.w4, gap2);
      cnt += count_chunk<KIND, CHECKED>(after2, (int32_t)(E2 - gap2), kept2_lo, kept2_hi, rem_end2, n_luts,
                                        batch.err);
    }

    if (PRIO) __builtin_amdgcn_s_setprio(0);
    // store the previous tile.  Its sign|mantissa registers are taken here,
    // once and on every path: the wait leaves the next step's stream words
    // in flight, and the store pass starts with no other load outstanding.
#pragma unroll
    for (uint32_t k = 0; k < kPrefetch; k++) asm volatile("" ::"v"(smv[k].x), "v"(smv[k].y));
    if constexpr (KIND == DF_KIND_BF16) {
      if (have_prev)
        store_tile<KIND>(jb, buf, prev_a, prev_lo, prev_hi, prev_he, prev_ng, prev_dirty, smv, lane);
      have_prev = active;
      prev_a = a;
      prev_lo = lo_r;
      prev_hi = hi_r;
      prev_he = hi_r + (hi < jb.n ? 1u : 0u);
      prev_ng = ngroups;
    }

    // prefix sum of the counts over the tile's 256 lanes
    const uint32_t wid = tid >> 6;
    const uint32_t x = wave_inclusive_sum(cnt);
    // (uint8 and uint4: two sets of sums, by step parity: their steps end
    // without a barrier, so a wave may write next step's sums while another
    // still reads these)
    const uint32_t wset = KIND != DF_KIND_BF16 ? 4 * groups * par : 0u;
    if ((tid & 63) == 63) wsum[wset + wid] = x;
    if (dyn && tid == 0) {  // last step's grab, for the workgroup: its first tile
      uint32_t pub = 0xFFFFFFFFu;  // no tile: past any span index
      if (grabbed) {
        if (tk == nx_lds[6]) nx_lds[7] |= 16;  // the counter's last value: freed at exit
        // a grab past the last unit gives a tile past the end; clamp so the
        // product cannot wrap into the span range
        const uint64_t t = (uint64_t)groups * (nx_lds[4] + (uint64_t)nx_lds[5] * tk);
        pub = t < 0xFFFFFFFFu ? (uint32_t)t : 0xFFFFFFFFu;
      }
      nx_lds[0] = pub;
    }
    __syncthreads();
    // the workgroup's first tile two steps ahead, then the grab for three
    // steps ahead (system scope: past the per-XCD L2 caches)
    uint32_t base_nxt2 = 0;
    if constexpr (kDynamic<KIND>) {
      base_nxt2 = base_nxt + step;
      if (dyn && !first_step) base_nxt2 = __builtin_amdgcn_readfirstlane(nx_lds[0]);
      first_step = false;
      grabbed = dyn && base_nxt2 < n_spans;
      if (grabbed && tid == 0) {
        if (nx_lds[1] == kNoTicket && !(nx_lds[7] & 32)) {  // slot not known yet (first grab)
          const uint32_t sl = find_slot(jb.ticket, ((uint64_t)nx_lds[9] << 32) | nx_lds[8]);
          nx_lds[1] = sl;
          if (sl == kNoTicket) {  // no slot found: deal every unit to itself
            nx_lds[4] = 3 * jb.wg_count;
            nx_lds[5] = 1;
            nx_lds[6] = 0xFFFFFFFFu;
            nx_lds[7] = 32;
          } else {
            const uint64_t cp = (uint64_t)(uintptr_t)slot_counter(sl, nx_lds[7] & 15);
            nx_lds[2] = (uint32_t)cp;
            nx_lds[3] = (uint32_t)(cp >> 32);
          }
        }
        uint32_t *ctr = (uint32_t *)(uintptr_t)(((uint64_t)nx_lds[3] << 32) | nx_lds[2]);
        tk = ctr ? __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) : tk + 1;
      }
    }
    const lds_u32 *ws = wsum + wset + 4 * grp;
    const uint32_t s0 = ws[0], s1 = ws[1], s2 = ws[2], s3 = ws[3];
    // the wave's index in its group; read as a uniform value in the BF16
    // kernel, whose compares on it were lane masks kept across the loop
    const uint32_t wq = (KIND == DF_KIND_BF16 ? __builtin_amdgcn_readfirstlane(wid) : wid) & 3;
    const uint32_t off = (wq > 0 ? s0 : 0u) + (wq > 1 ? s1 : 0u) + (wq > 2 ? s2 : 0u) + x - cnt;
    if (CHECKED && active && lane == 0 && s0 + s1 + s2 + s3 != hi_r - lo_r)
      atomicOr(batch.err, DF_DEVERR_COUNT);
    if constexpr (KIND == DF_KIND_U4) {  // the previous tile (its phase 2 ended before the scan barrier)
      if (have_prev)
        store_tile<KIND>(jb, pbuf, prev_a, prev_lo, prev_hi, prev_he, prev_ng, prev_dirty, smv, lane);
      have_prev = active;
      prev_a = a;
      prev_lo = lo_r;
      prev_hi = hi_r;
      prev_he = hi_r + (hi < jb.n ? 1u : 0u);
      prev_ng = ngroups;
    }
    {  // staging bytes phase 2 may write: every lane ends by lo_r + off + cnt
       // + the slack (uint4: nibbles, two per byte)
      const uint32_t e = lo_r + s0 + s1 + s2 + s3 + kSlack<KIND>;
      const uint32_t d = ((KIND == DF_KIND_U4 ? (e + 1) / 2 : e) + 7) & ~7u;
      prev_dirty = d < out_bytes ? d : out_bytes;
    }

    if (PRIO) __builtin_amdgcn_s_setprio(3);
    // phase 2: walk the same entries again (those phase 1 kept are replayed
    // from registers, the rest decoded again) and OR their symbol bytes into
    // the staging buffer until the lane's cnt codes are written.  The entry
    // that crosses the chunk end is not clipped: its codes past the end are
    // the next lane's first codes (code boundaries are a property of the
    // stream), written to the same positions with the same values by that
    // lane, so the OR (the uint8 store) is idempotent; past the tile's last
    // code they land in the staging slack, which is never stored.  A lane
    // whose codes would not fit the buffer (only with corrupt offsets or
    // stream) skips the phase, so LDS writes stay inside the buffer.
    {
      // staging positions: bytes, uint4 nibbles (two per byte)
      const uint32_t cap = KIND == DF_KIND_U4 ? 2 * out_bytes : out_bytes;
      uint32_t q = (KIND == DF_KIND_U4 ? 2 * buf : buf) + lo_r + off;
      uint32_t qend = q + cnt;
      // (each term is bounded first, so the sum cannot wrap even when a
      // damaged table makes the counts meaningless)
      const bool fits = off <= cap && cnt <= cap && lo_r + off + cnt + kSlack<KIND> <= cap;
      if (!fits) {
        qend = q;
        if (CHECKED) atomicOr(batch.err, DF_DEVERR_COUNT);
      }
      if constexpr (C == 2) {  // the first chunk's codes, then the second's
        const uint32_t q1 = q + cnt1 < qend ? q + cnt1 : qend;
        write_chunk<KIND, CHECKED>(q, q1, after, kept_lo, kept_hi, n_luts, batch.err);
        q = write_chunk<KIND, CHECKED>(q1, qend, after2, kept2_lo, kept2_hi, n_luts, batch.err);
      } else {
        q = write_chunk<KIND, CHECKED>(q, qend, after, kept_lo, kept_hi, n_luts, batch.err);
      }
      // uint4: a tile that ends at an odd element shares its last output
      // byte with the next tile, and writes that whole byte, so it needs the
      // next tile's first symbol at staging position hi_r.  The lane with
      // the tile's last code has it from its last lookup's lookahead (q
      // moved past qend) or, when that lookup ended exactly on a code
      // boundary, decodes it here: the code starts E - rem_end bits into
      // the lane's 128 bits (it is the lane's walk end, at most 31 bits past
      // the chunk, so its 32-bit window lies inside them).
      if (KIND == DF_KIND_U4 && fits && cnt > 0 && off + cnt == s0 + s1 + s2 + s3 && (hi & 1) &&
          hi < jb.n && q == qend) {
        const uint32_t p = E - (uint32_t)rem_end;
        const uint32_t win = p >= 64 ? __builtin_amdgcn_alignbit(cur.w3, cur.w2, p - 64)
                           : p >= 32 ? __builtin_amdgcn_alignbit(cur.w2, cur.w1, p - 32)
                                     : __builtin_amdgcn_alignbit(cur.w1, cur.w0, p);
        const uint32_t c = long_code<KIND, CHECKED>(n_luts, win, batch.err);
        __hip_atomic_fetch_or(lds<lds_u32>((q >> 3) << 2), (c & 0xFu) << ((q & 7) * 4), __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
    if constexpr (KIND == DF_KIND_U8) {
      // uint8: each wave stores its own output range as soon as its phase 2
      // is done.  Its lanes' codes are output elements [r0, r1) of the span,
      // staged by this wave (a neighbour's lookahead writes bytes of the
      // range with the same values), so the store needs no barrier; the
      // next step's phase 2 writes staging only after the scan barrier,
      // which every wave reaches after its store, and the sums are read
      // from the other set next step.  Against the group's store pass one
      // step late (with its end-of-step barrier), and with the range's
      // partial first and last granules stored one byte per lane rather
      // than byte by byte in one lane, the uint8 block went from 195 to
      // 171 us side by side.  The store runs at the base priority (at the
      // decode's it was 5% slower).
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      if (PRIO) __builtin_amdgcn_s_setprio(0);
      if (active) {
        const uint32_t tot = hi_r - lo_r;
        uint32_t w0 = (wq > 0 ? s0 : 0u) + (wq > 1 ? s1 : 0u) + (wq > 2 ? s2 : 0u);
        uint32_t w1 = w0 + (wq == 0 ? s0 : wq == 1 ? s1 : wq == 2 ? s2 : s3);
        // (damaged counts: each bound limited to the span first)
        w0 = w0 < tot ? w0 : tot;
        w1 = w1 < tot ? (w1 < w0 ? w0 : w1) : tot;
        const uint32_t r0 = lo_r + w0, r1 = lo_r + w1;
        uint8_t *dst_t = (uint8_t *)jb.dst + a;
        const lds_v4 *ex_t = lds<const lds_v4>(buf);
        const uint32_t l = lane & 63;
        // the granules wholly inside [r0, r1): one 16-byte store each
        const uint32_t fs = (r0 + 15) / 16, fe = r1 / 16;
        for (uint32_t g = fs + l; g < fe; g += 64) *(v4u *)(dst_t + 16 * g) = ex_t[g];
        // the bytes of the first and last granule that are not whole: one
        // byte per lane, lanes 0..15 the first granule, 16..31 the last
        if (l < 32 && r0 < r1) {
          const uint32_t p = 16 * (l < 16 ? r0 / 16 : (r1 - 1) / 16) + (l & 15);
          if (p >= r0 && p < r1 && (p < 16 * fs || p >= 16 * fe)) dst_t[p] = *lds<const lds_u8>(buf + p);
        }
      }
    } else if constexpr (kBufs<KIND> == 1) {
      __syncthreads();
    }
    par ^= 1u;
    if constexpr (kDynamic<KIND>) {
      base = base_nxt;
      base_nxt = base_nxt2;
    } else {
      base += step;
    }
  }
  // a workgroup that took its counter's last value counts it finished (the
  // last counter of the slot to finish frees the slot)
  if (dyn && tid == 0 && (nx_lds[7] & 16) && nx_lds[1] != kNoTicket) counter_finished(nx_lds[1], nx_lds[10]);
  // the last tile of this group (BF16 and uint4)
  if constexpr (KIND != DF_KIND_U8) {
    if (kBufs<KIND> == 2) __syncthreads();  // (the loop's exit is uniform over the workgroup)
    if (have_prev) {
      uint2 smv[kPrefetch];
#pragma unroll
      for (uint32_t k = 0; k < kPrefetch; k++) {
        const uint32_t g = lane + k * kTPB;
        smv[k] = KIND == DF_KIND_BF16 && g < prev_ng ? *(const uint2 *)(jb.sm + prev_a + 8 * (uint64_t)g)
                                                      : make_uint2(0, 0);
      }
#pragma unroll
      for (uint32_t k = 0; k < kPrefetch; k++) asm volatile("" ::"v"(smv[k].x), "v"(smv[k].y));
      store_tile<KIND>(jb, buf0 + (kBufs<KIND> == 2 ? (par ^ 1u) * out_bytes : 0u), prev_a, prev_lo, prev_hi,
                       prev_he, prev_ng, prev_dirty, smv, lane);
    }
  }
}

// ------------------------------------------------------------------ host side
struct DeviceProps {
  bool ready;
  int dev;
  int cus;
  int max_lds;
};
constexpr int kMaxDevices = 64;
DeviceProps g_props[kMaxDevices];
std::mutex g_mu;

typedef void (*KernelFn)(const Batch);
template <int KIND>
KernelFn kernel_of(bool checked, bool prio) {
  if (checked) return prio ? decode_kernel<KIND, true, true> : decode_kernel<KIND, true, false>;
  return prio ? decode_kernel<KIND, false, true> : decode_kernel<KIND, false, false>;
}

KernelFn kernel_for(df_kind kind, bool checked, bool prio) {
  if (kind == DF_KIND_BF16) return kernel_of<DF_KIND_BF16>(checked, prio);
  if (kind == DF_KIND_U4) return kernel_of<DF_KIND_U4>(checked, prio);
  return kernel_of<DF_KIND_U8>(checked, prio);
}

df_status device_props(DeviceProps *out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DF_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_mu);
  DeviceProps &p = g_props[dev];
  if (!p.ready) {
    p.dev = dev;
    if (hipDeviceGetAttribute(&p.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipDeviceGetAttribute(&p.max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
      return DF_ERR_HIP;
    // allow dynamic LDS up to the device limit; where the runtime needs no
    // opt-in the call may fail, which is harmless, so its error is cleared
    const df_kind kinds[3] = {DF_KIND_BF16, DF_KIND_U8, DF_KIND_U4};
    for (df_kind k : kinds)
      for (int c = 0; c < 4; c++)
        if (hipFuncSetAttribute((const void *)kernel_for(k, (c & 1) != 0, (c & 2) != 0),
                                hipFuncAttributeMaxDynamicSharedMemorySize, p.max_lds - 64) != hipSuccess)
          (void)hipGetLastError();
    p.ready = true;
  }
  *out = p;
  return DF_OK;
}

// Resident workgroups per CU for a kernel, block size and LDS size, asked of
// the runtime once per device and kept (the query costs tens of microseconds
// of host time, which a launch of a small container would otherwise pay).
struct OccEntry {
  int dev;
  KernelFn fn;
  int threads;
  size_t lds;
  int occ;
};
constexpr int kOccCache = 256;
OccEntry g_occ[kOccCache];
int g_occ_n = 0;

df_status occupancy(int dev, KernelFn fn, int threads, size_t lds, int *occ) {
  {
    std::lock_guard<std::mutex> lk(g_mu);
    for (int i = 0; i < g_occ_n; i++)
      if (g_occ[i].dev == dev && g_occ[i].fn == fn && g_occ[i].threads == threads && g_occ[i].lds == lds) {
        *occ = g_occ[i].occ;
        return DF_OK;
      }
  }
  int o = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, (const void *)fn, threads, lds) != hipSuccess) return DF_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_occ_n < kOccCache) g_occ[g_occ_n++] = {dev, fn, threads, lds, o};
  *occ = o;
  return DF_OK;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

df_status check_view(const df_device_view *v, const void *dst) {
  if (!v || (v->kind != DF_KIND_BF16 && v->kind != DF_KIND_U8 && v->kind != DF_KIND_U4)) return DF_ERR_ARG;
  if (v->n == 0) return DF_OK;
  if (!dst || !aligned(dst, 16)) return DF_ERR_ARG;
  if (!v->bitstream || !v->gaps || !v->tile_out || !v->lut || !v->dtab) return DF_ERR_ARG;
  if (v->kind == DF_KIND_BF16 && (!v->sign_mantissa || !aligned(v->sign_mantissa, 8))) return DF_ERR_ARG;
  if (!aligned(v->bitstream, 8) || !aligned(v->gaps, 4) || !aligned(v->tile_out, 8) ||
      !aligned(v->lut, 16) || !aligned(v->dtab, 16))
    return DF_ERR_ARG;
  if (v->n_tiles == 0 || v->n_tiles >= (1ull << 31) || v->n_threads == 0 ||
      v->n_threads > v->n_tiles * DF_THREADS_PER_TILE ||
      v->n_threads <= (v->n_tiles - 1) * DF_THREADS_PER_TILE)
    return DF_ERR_ARG;
  if (v->total_bits <= (v->n_threads - 1) * 64 || v->total_bits > v->n_threads * 64 + DF_MAX_LEN)
    return DF_ERR_ARG;
  if (v->n_luts < 1 || v->n_luts > DF_MAX_LUTS) return DF_ERR_ARG;
  if (v->max_tile_elems < 1 || v->max_tile_elems > DF_TILE_BITS) return DF_ERR_ARG;
  return DF_OK;
}

uint32_t out_bytes_for(df_kind kind, uint32_t max_tile_elems) {
  if (kind == DF_KIND_U4)  // nibbles: range rounded down to 32 elements, the element after it,
                           // slack, rounded to 32, one spare granule; two per byte
    return (((max_tile_elems + 31 + 1 + kSlack<DF_KIND_U4> + 31) & ~31u) + 32) / 2;
  // tile range rounded down to a 16-element granule, plus the slack of the
  // last lane's lookahead writes, rounded to 16, plus one spare granule
  return ((max_tile_elems + 15 + kSlack<DF_KIND_BF16> + 15) & ~15u) + 16;
}

// The first-choice counter slot of a dynamically scheduled job.  Launches
// take hints in turn, so that jobs in flight at once usually claim their
// hinted slot at the first try; the device settles the claim either way.
std::atomic<uint32_t> g_hint{0};
uint32_t ticket_slot() { return g_hint.fetch_add(1) % kTicketSlots; }

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
  // a capped launch (any view with a workgroup cap) keeps its waves at the
  // base priority
  bool capped = false;
  for (uint32_t i = 0; i < count; i++) capped = capped || views[i].max_workgroups != 0;
  KernelFn fn = kernel_for(kind, checked, !capped);

  for (uint32_t base = 0; base < count; base += DF_MAX_BATCH) {
    const uint32_t m = count - base < DF_MAX_BATCH ? count - base : DF_MAX_BATCH;
    Batch b;
    memset(&b, 0, sizeof b);
    // tiles per lane group and step: kChunks for the kind
    const uint32_t span_tiles = kind == DF_KIND_U8 ? kChunks<DF_KIND_U8> : 1u;
    uint32_t max_elems = 0, max_luts = 1;
    uint64_t spans = 0;
    uint32_t nj = 0;
    uint32_t idx[DF_MAX_BATCH];
    for (uint32_t i = 0; i < m; i++) {
      const df_device_view &v = views[base + i];
      if (v.n == 0) continue;
      idx[nj++] = base + i;
      spans += (v.n_tiles + span_tiles - 1) / span_tiles;
      if (v.max_tile_elems > max_elems) max_elems = v.max_tile_elems;
      if (v.n_luts > max_luts) max_luts = v.n_luts;
    }
    if (nj == 0) continue;
    const uint32_t out_bytes = out_bytes_for(kind, span_tiles * max_elems);
    const uint32_t lut_bytes = max_luts * 512;
    // tile groups per workgroup: the choice that keeps the most waves
    // resident per CU (LDS is the limit: the tables are shared per workgroup)
    uint32_t groups = 0;
    int per_cu = 0;
    size_t lds = 0;
    for (uint32_t g = kMaxGroups; g >= 1; g--) {
      const size_t need = (size_t)(kind == DF_KIND_U8 ? kTabBytes<DF_KIND_U8> : kDtabBytes) + lut_bytes +
                          (size_t)g * out_bytes * (kind == DF_KIND_U4 ? kBufs<DF_KIND_U4> : 1u) + 32 * g + 64;
      if (need > (size_t)props.max_lds) continue;
      int occ = 0;
      if (occupancy(props.dev, fn, (int)(g * kTPB), need, &occ) != DF_OK) return DF_ERR_HIP;
      if (occ < 1) continue;
      if (groups == 0 || (uint64_t)occ * g > (uint64_t)per_cu * groups) {
        groups = g;
        per_cu = occ;
        lds = need;
      }
    }
    if (groups == 0) return DF_ERR_ARG;
    uint64_t budget = (uint64_t)props.cus * (uint64_t)per_cu;
    for (uint32_t k = 0; k < nj; k++) {  // the caller's cap, if any
      const uint32_t cap = views[idx[k]].max_workgroups;
      if (cap && cap < budget) budget = cap;
    }
    if (budget < nj) budget = nj;
    uint32_t wg = 0;
    for (uint32_t k = 0; k < nj; k++) {
      const df_device_view &v = views[idx[k]];
      const uint64_t v_spans = (v.n_tiles + span_tiles - 1) / span_tiles;
      uint64_t share = budget * v_spans / spans;
      const uint64_t need = (v_spans + groups - 1) / groups;
      if (share < 1) share = 1;
      if (share > need) share = need;
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
      jb.ticket = kNoTicket;
      if (kind == DF_KIND_BF16 && v.n_tiles > 3 * share * groups && v.n_tiles < (1ull << 31))
        jb.ticket = ticket_slot();
      wg += (uint32_t)share;
    }
    b.count = nj;
    b.lut_bytes = lut_bytes;
    b.out_bytes = out_bytes;
    b.err = err;
    hipLaunchKernelGGL(fn, dim3(wg), dim3(groups * kTPB), lds, stream, b);
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
