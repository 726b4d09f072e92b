// Continuous weight streaming for the expert GEMMs (one workgroup = 4 wavefronts).
//
// Work items are (row group, expert, quad of column tiles); the 4 wavefronts of a
// workgroup take the 4 tiles of a quad, so they share one expert, one row group and one
// activation slice.  A workgroup owns a strided subset of the items and walks them
// back to back:
//
//   weights   each wave keeps a register ring of one step: SPS segments (a segment = 256
//             K values of NS x 16 rows).  A segment's registers are reloaded with the same
//             segment of the next step as soon as they have been copied into the LDS
//             transpose slab, so about one step of loads is always in flight while the
//             wave computes.  The ring runs across item boundaries, so there is no
//             pipeline drain between items.
//   scales    staged per wave in LDS, one run of SRUN segments at a time: one coalesced
//             16-byte load per lane brings the run's scales of all NS x 16 rows (the
//             lanes of ScaleRun::LANES_PER_ROW cover one row), one step ahead of use, and each segment
//             reads its row's 8 bytes back with one LDS load.  Loading 16 bytes of one row
//             per lane and segment pair instead made the scale requests, not the bytes, cost
//             a seventh of the kernel's time.
//   acts      the activation rows of an item are staged in LDS, chunk by chunk, shared
//             by the 4 waves.  A chunk holds CS segments of the item's R rows, with
//             CS = (row-segments per chunk) / R rounded down to a multiple of SPS (at least
//             SPS), so a chunk fits the kernel's chunk buffer, is loaded by whole rounds of
//             16-byte loads of the 256 threads, and ends on a step.  The loads of chunk i+1 are issued when
//             chunk i starts and written to the other LDS buffer when it ends; LDS counters
//             hand it over.
//
// Loads retire in issue order and every step issues the same weight loads (an exhausted
// cursor re-reads its last segment), so the compiler's waits stay exact: a segment waits
// only for its own loads, issued one step earlier.
//
// MXFP8 activations (policies with ACT8): each thread quantizes its 16-byte piece of bf16
// activations as it stores it into the chunk buffer (the 4 pieces of a 32-value block are
// 4 consecutive threads), and segments go to the scaled MFMA with the weights' codes and
// scales as they are (mx_act8.hpp).
#pragma once
#include "mx_act8.hpp"
#include "mx_device.hpp"

namespace mx {

constexpr int WG_WAVES = 4;
// sched_barrier mask: ALU, VALU, SALU, MFMA, all DS and transcendental instructions may be
// scheduled across; vector memory instructions may not
constexpr int SCHED_ALL_BUT_VMEM = 0x1 | 0x2 | 0x4 | 0x8 | 0x80 | 0x100 | 0x200 | 0x400;
// Activation chunk geometry for a chunk buffer of BYTES (one of two per workgroup):
// R rows x CS segments x 512 B, loaded in ROUNDS rounds of one 16-byte piece per thread.
template <int BYTES>
struct XGeom {
  static constexpr int PIECES = BYTES / 16;
  static constexpr int ROUNDS = PIECES / (WG_WAVES * 64);
  static constexpr int ROWSEGS = BYTES / (SEG_K * 2);  // row-segments a chunk holds
  static_assert(ROUNDS * WG_WAVES * 64 == PIECES, "whole rounds");
  static_assert(ROWSEGS <= 64, "the reciprocal quotient below is exact only below 64 row-segments");
};

// Activation chunk length, in segments, for a group of `rows` rows in a chunk of `rowsegs`
// row-segments: as many segments as fit, a multiple of `align` (the weight step, so chunks
// end on steps), and at least one step.
__host__ __device__ constexpr int chunk_segments(int rows, int nseg, int align, int rowsegs) {
  return (rowsegs / rows / align * align) < align ? align
         : ((rowsegs / rows / align * align) < nseg ? rowsegs / rows / align * align : nseg);
}

// Scale staging: runs of SRUN segments (an item's segment count must be a multiple).  A
// run of one row is SRUN * 8 bytes; a lane loads LOAD of them (16, or 8 for one-segment
// runs), so LANES_PER_ROW lanes cover a row and one wave load covers ROWS_PER_LOAD rows.
// A wave's NS x 16 rows need loads<NS>() loads; the last one may cover fewer rows than a
// full load, its other lanes repeat rows and do not store.
template <bool C, class A, class B>
struct pick_type {
  typedef A type;
};
template <class A, class B>
struct pick_type<false, A, B> {
  typedef B type;
};
template <int SRUN_>
struct ScaleRun {
  static constexpr int SRUN = SRUN_;
  static constexpr int ROW_BYTES = SRUN * SEG_SCALES;
  static constexpr int LOAD = ROW_BYTES < 16 ? ROW_BYTES : 16;
  static constexpr int LANES_PER_ROW = ROW_BYTES / LOAD;
  static constexpr int ROWS_PER_LOAD = 64 / LANES_PER_ROW;
  typedef typename pick_type<LOAD == 16, u32x4, u32x2>::type Reg;
  static_assert(LOAD == 16 || LOAD == 8, "8- or 16-byte scale loads");
  template <int NS>
  static constexpr int loads() {
    static_assert((NS * SUB_ROWS) % ROWS_PER_LOAD == 0 || NS * SUB_ROWS < ROWS_PER_LOAD, "whole scale loads");
    return (NS * SUB_ROWS + ROWS_PER_LOAD - 1) / ROWS_PER_LOAD;
  }
  template <int NS>
  static constexpr int slab_bytes() {
    return NS * SUB_ROWS * ROW_BYTES;
  }
};
constexpr int SRUN = 4;  // the run of the gate_up GEMM and of down when I % 1024 == 0
typedef ScaleRun<SRUN> ScaleRun4;

// One step of the weight ring: SPS consecutive segments of the wave's NS subtiles.
template <int NS, int SPS>
struct WRing {
  u32x4 w[SPS][NS][2];
};

// Position in a workgroup's work: the item `it`, and its ordinal n among the workgroup's
// first-group items (-1 while it streams extra row groups, which come first).
struct ItemPos {
  int n, it;
};

template <int NS, class SR>
struct WCursor {
  ItemPos at;  // current item
  int seg;  // first segment of the step the ring is reloaded with
  const uint8_t* w[NS][2];                      // this lane's code bytes of segment 0 (2 rows)
  const uint8_t* sr[SR::template loads<NS>()];  // this lane's scale bytes of segment 0, per load
};

// Fill the ring with the step at cursor c, in the order the loop reloads it, so that the
// compiler's waits on entry to the loop match its waits inside it.
template <int NS, int SPS, class SR>
__device__ __forceinline__ void wring_load(WRing<NS, SPS>& r, const WCursor<NS, SR>& c) {
#pragma unroll
  for (int j = 0; j < SPS; ++j) {
    const size_t wo = (size_t)(c.seg + j) * SEG_BYTES;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      r.w[j][i][0] = ld_stream16(c.w[i][0] + wo);
      r.w[j][i][1] = ld_stream16(c.w[i][1] + wo);
    }
    __builtin_amdgcn_sched_barrier(SCHED_ALL_BUT_VMEM);
  }
}

// Scales of the run starting at c.seg (a multiple of SRUN), one load per lane and load.
template <int NS, class SR>
__device__ __forceinline__ void srun_load(typename SR::Reg (&sreg)[SR::template loads<NS>()], const WCursor<NS, SR>& c) {
#pragma unroll
  for (int k = 0; k < SR::template loads<NS>(); ++k)
    sreg[k] = *reinterpret_cast<const typename SR::Reg*>(c.sr[k] + (size_t)c.seg * SEG_SCALES);
  __builtin_amdgcn_sched_barrier(SCHED_ALL_BUT_VMEM);
}

// The slab holds row rho = i * 16 + r of the run at rho * ROW_BYTES; a load's 64 lanes cover
// ROWS_PER_LOAD consecutive rows, so lane l of load k lands at (k * 64 + l) * LOAD.
template <int NS, class SR>
__device__ __forceinline__ void srun_store(uint8_t* __restrict__ sslab,
                                           const typename SR::Reg (&sreg)[SR::template loads<NS>()], int lane) {
#pragma unroll
  for (int k = 0; k < SR::template loads<NS>(); ++k)
    if (k * 64 + lane < NS * SUB_ROWS * SR::LANES_PER_ROW)
      *reinterpret_cast<typename SR::Reg*>(sslab + (k * 64 + lane) * SR::LOAD) = sreg[k];
}

// What the kernels need of an item; all fields are uniform across the workgroup.
struct ItemInfo {
  int e;      // expert
  int row0;   // sorted position of the group's first row
  int rows;   // rows in the group (1..16)
  int tile0;  // first column tile of the quad
  int cs;     // activation chunk length in segments
};

// Per-workgroup cursor over activation chunks.
struct XChunk {
  ItemPos at;  // item
  int c0;  // first segment of the chunk within the item
  int ns;  // segments in the chunk
  ItemInfo info;
};

// LDS byte offset of the 16-byte piece p (0..31) of row m of segment s of a chunk with R
// rows; pieces are XOR-swizzled by row so 16 lanes reading 16 rows hit distinct banks.
__device__ __forceinline__ uint32_t xpiece_off(int s, int m, int R, int p) {
  return (uint32_t)(((s * R + m) * 32 + (p ^ (m & 31))) * 16);
}

// Chunk hand-off without a workgroup barrier.  Each thread stores its pieces of chunk i+1
// into buffer (i+1) % 2 and then adds 1 to that buffer's LDS counter; a wave starts chunk
// i+1 once the counter shows all WG_THREADS threads of that generation.  (The count is
// per thread, not per wave: the compiler merges the adds of a wave's lanes into one add
// of the lane count, so the total is the same either way.)  Because starting chunk i
// needed every thread's pieces of chunk i, written after its wave finished chunk i-1, no
// wave is ever more than one chunk ahead of another: the buffer being written is never
// the one still being read, and two buffers suffice.
//
// Ordering: the wave waits for its own LDS stores (lgkmcnt, which does not count global
// loads) before the counter update, and a reader's data loads are issued after its
// counter load returned.  The compiler is kept from moving LDS accesses across the
// hand-off by the asm memory clobbers; a workgroup-scope release/acquire would also wait
// for the wave's outstanding global loads and drain the weight stream.
constexpr uint32_t WG_THREADS = WG_WAVES * 64;

__device__ __forceinline__ void xready_publish(uint32_t* ctr) {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt left at their maximum
  __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ void xready_wait(const uint32_t* ctr, uint32_t target) {
  while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target) __builtin_amdgcn_s_sleep(1);
  __asm__ volatile("" ::: "memory");
}

// Row-segment rs (< 64) of a chunk with R rows is segment rs / R, row rs % R.
// The quotient is (rs * ceil(2^16 / R)) >> 16, exact for rs < 64 and R <= 16.
__device__ __forceinline__ uint32_t rows_reciprocal(int R) { return (65536u + (uint32_t)R - 1u) / (uint32_t)R; }

// Issue the activation loads of chunk `ch`: XROUNDS rounds of one 16-byte piece per thread
// (threads past the chunk repeat its last piece; skipping the unneeded rounds costs more
// registers than the loads it saves).  Lane m < 16 holds row m's element offset, and each
// thread fetches its row's offset from there with one cross-lane read.
// COHERENT: device-coherent loads instead of the policy's (the reload of a chunk that another
// workgroup of the launch may have written since a cached copy was fetched)
template <bool COHERENT = false, int XROUNDS, class P>
__device__ __forceinline__ void xchunk_load(const P& p, const XChunk& ch, u32x4 (&xv)[XROUNDS], int tid) {
  const int R = ch.info.rows;
  const int npieces = R * ch.ns * 32;
  const uint32_t inv = rows_reciprocal(R);
  int myoff = 0;  // lane (tid & 15)'s row offset
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const int off = (m < R) ? p.x_row_offset(ch.info, m) : 0;
    myoff = ((tid & 15) == m) ? off : myoff;
  }
#pragma unroll
  for (int r = 0; r < XROUNDS; ++r) {
    const int q = min(r * (WG_WAVES * 64) + tid, npieces - 1);
    const int rs = q >> 5, pc = q & 31;
    const int s = (int)(((uint32_t)rs * inv) >> 16), m = rs - s * R;
    const int ro = __builtin_amdgcn_ds_bpermute(m << 2, myoff);
    const uint16_t* a = p.xact + (size_t)ro + (size_t)(ch.c0 + s) * SEG_K + pc * 8;
    xv[r] = COHERENT ? ld16_coherent(a) : p.xload(a);
  }
}

template <int XROUNDS>
__device__ __forceinline__ void xchunk_store(uint8_t* __restrict__ buf, const XChunk& ch, const u32x4 (&xv)[XROUNDS],
                                             int tid) {
  const int R = ch.info.rows;
  const int npieces = R * ch.ns * 32;
  const uint32_t inv = rows_reciprocal(R);
#pragma unroll
  for (int r = 0; r < XROUNDS; ++r) {
    const int q = min(r * (WG_WAVES * 64) + tid, npieces - 1);
    const int rs = q >> 5, pc = q & 31;
    const int s = (int)(((uint32_t)rs * inv) >> 16), m = rs - s * R;
    *reinterpret_cast<u32x4*>(buf + xpiece_off(s, m, R, pc)) = xv[r];
  }
}

// MXFP8 chunk layout (ACT8): the 256 code bytes of row-segment (s, m) at (s * R + m) * 256,
// as 16 pieces of 16 bytes XOR-swizzled by row (piece c at ((c ^ (m & 15)) << 4)), and its 8
// scale bytes at XCHUNK / 2 + (s * R + m) * 8 (a chunk holds at most XCHUNK / 512
// row-segments, so both halves fit).  Threads past the chunk quantize a repeat of its last
// piece and store nothing: their block maximum would not be the block's.
template <int XROUNDS, int XCHUNK>
__device__ __forceinline__ void xchunk_store_a8(uint8_t* __restrict__ buf, const XChunk& ch,
                                                const u32x4 (&xv)[XROUNDS], int tid) {
  const int R = ch.info.rows;
  const int npieces = R * ch.ns * 32;
  const uint32_t inv = rows_reciprocal(R);
#pragma unroll
  for (int r = 0; r < XROUNDS; ++r) {
    const int q0 = r * (WG_WAVES * 64) + tid;
    const int q = min(q0, npieces - 1);
    const int rs = q >> 5, pc = q & 31;
    const int s = (int)(((uint32_t)rs * inv) >> 16), m = rs - s * R;
    uint32_t sb;
    const u32x2 c = act8_quant_quad(xv[r], sb);
    if (q0 < npieces) {
      const int row = s * R + m;
      *reinterpret_cast<u32x2*>(buf + row * 256 + (((pc >> 1) ^ (m & 15)) << 4) + (pc & 1) * 8) = c;
      if ((pc & 3) == 0) buf[XCHUNK / 2 + row * 8 + (pc >> 2)] = (uint8_t)sb;
    }
  }
}

template <int XROUNDS, int XCHUNK, bool A8>
__device__ __forceinline__ void xchunk_put(uint8_t* __restrict__ buf, const XChunk& ch, const u32x4 (&xv)[XROUNDS],
                                           int tid) {
  if constexpr (A8)
    xchunk_store_a8<XROUNDS, XCHUNK>(buf, ch, xv, tid);
  else
    xchunk_store<XROUNDS>(buf, ch, xv, tid);
}

// Activations written earlier in the same launch (policies with SENTINEL, down after gate_up
// in one launch): every h element holds 0xFFFF until gate_up writes it, with a device-coherent
// store, and gate_up writes each element once.  So any other value a load returns, from
// memory or from a cached copy, is the element's final value, and the chunk's loads can be
// ordinary cached ones.  A wave that finds an 0xFFFF in its pieces (not yet written when the
// copy was fetched, or a NaN that happens to have that pattern) waits until every workgroup
// has finished its gate_up items (p.wait_all_written) and loads its pieces again with
// device-coherent loads, which do not return a stale cached copy.  The branch is
// wave-uniform, and ends with all of the wave's loads complete, so the waits the compiler
// counts on the common path stay exact.
template <class P, int XROUNDS>
__device__ __forceinline__ void xchunk_settle(const P& p, const XChunk& ch, u32x4 (&xv)[XROUNDS], int tid) {
  if constexpr (P::SENTINEL) {
    bool unwritten = false;
#pragma unroll
    for (int r = 0; r < XROUNDS; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) unwritten |= (xv[r][c] & 0xFFFFu) == 0xFFFFu || (xv[r][c] >> 16) == 0xFFFFu;
    if (__ballot(unwritten) != 0ull) {
      p.wait_all_written();
      xchunk_load<true>(p, ch, xv, tid);
      __asm__ volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    }
  }
}

// Consume one segment: LDS transpose of the codes, decode, MFMA with activations from the
// chunk buffer (xrow: this lane's row within the chunk; rows past R read row 0, whose
// products land in output columns that are not stored).  The scales come from the wave's
// scale slab (segment u of the staged run).  Once the codes are in the slab, w is reloaded
// with segment `nseg_next` of the cursor `c` (the same segment of the next step).
template <int NS, class SR>
__device__ __forceinline__ void segment_compute(u32x4 (&w)[NS][2], const uint8_t* __restrict__ sslab, int u,
                                                const WCursor<NS, SR>& c, int nseg_next,
                                                const uint8_t* __restrict__ xbuf, int sl, int R, int xrow,
                                                uint8_t* __restrict__ slab, const uint32_t (&lds_wr)[2],
                                                const uint32_t (&lds_rd)[2], uint32_t sshift, int lane,
                                                f32x4 (&acc)[NS]) {
  // One slab serves the NS subtiles in turn: the wave's LDS accesses execute in order, so
  // subtile i+1's stores cannot overtake subtile i's loads.
  u32x4 wc[NS][2];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    *reinterpret_cast<u32x4*>(slab + lds_wr[0]) = w[i][0];
    *reinterpret_cast<u32x4*>(slab + lds_wr[1]) = w[i][1];
    wc[i][0] = *reinterpret_cast<const u32x4*>(slab + lds_rd[0]);
    wc[i][1] = *reinterpret_cast<const u32x4*>(slab + lds_rd[1]);
  }
  const size_t wo = (size_t)nseg_next * SEG_BYTES;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    w[i][0] = ld_stream16(c.w[i][0] + wo);
    w[i][1] = ld_stream16(c.w[i][1] + wo);
  }
  // Keep global loads in segment order (everything else may still move across), so the
  // next step's waits are progressive: segment j waits only for the loads of segment j.
  __builtin_amdgcn_sched_barrier(SCHED_ALL_BUT_VMEM);
  // the 8 scale bytes of subtile i's row (lane & 15) for this segment
  u32x2 sc2[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i)
    sc2[i] = *reinterpret_cast<const u32x2*>(sslab + (i * SUB_ROWS + (lane & 15)) * SR::ROW_BYTES + u * SEG_SCALES);
  const int j = lane >> 4;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float sc[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) sc[i] = e8m0_scale_operand((sc2[i][h] >> sshift) & 0xFFu);
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      const bf16x8 xb =
          as_bf16x8(*reinterpret_cast<const u32x4*>(xbuf + xpiece_off(sl, xrow, R, (j + 4 * h) * 4 + c4)));
#pragma unroll
      for (int i = 0; i < NS; ++i) acc[i] = mfma_bf16(decode8(wc[i][h][c4], sc[i]), xb, acc[i]);
    }
  }
}

// The same with MXFP8 activations: the codes go to the scaled MFMA undecoded with their
// scale bytes; the activation lane of group g reads pieces 8h + g and 8h + g + 4 of its row
// (half g & 1 of blocks 4h + (g >> 1) and 4h + 2 + (g >> 1)) and the scale of block 4h + g.
template <int NS, class SR, int XCHUNK>
__device__ __forceinline__ void segment_compute_a8(u32x4 (&w)[NS][2], const uint8_t* __restrict__ sslab, int u,
                                                   const WCursor<NS, SR>& c, int nseg_next,
                                                   const uint8_t* __restrict__ xbuf, int sl, int R, int xrow,
                                                   uint8_t* __restrict__ slab, const uint32_t (&lds_wr)[2],
                                                   const uint32_t (&lds_rd)[2], uint32_t sshift, int lane,
                                                   f32x4 (&acc)[NS]) {
  u32x4 wc[NS][2];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    *reinterpret_cast<u32x4*>(slab + lds_wr[0]) = w[i][0];
    *reinterpret_cast<u32x4*>(slab + lds_wr[1]) = w[i][1];
    wc[i][0] = *reinterpret_cast<const u32x4*>(slab + lds_rd[0]);
    wc[i][1] = *reinterpret_cast<const u32x4*>(slab + lds_rd[1]);
  }
  const size_t wo = (size_t)nseg_next * SEG_BYTES;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    w[i][0] = ld_stream16(c.w[i][0] + wo);
    w[i][1] = ld_stream16(c.w[i][1] + wo);
  }
  __builtin_amdgcn_sched_barrier(SCHED_ALL_BUT_VMEM);
  u32x2 sc2[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i)
    sc2[i] = *reinterpret_cast<const u32x2*>(sslab + (i * SUB_ROWS + (lane & 15)) * SR::ROW_BYTES + u * SEG_SCALES);
  const int g = lane >> 4;
  const int row = sl * R + xrow;
  const uint8_t* xr = xbuf + row * 256;
  const u32x2 xs2 = *reinterpret_cast<const u32x2*>(xbuf + XCHUNK / 2 + row * 8);
  const int sw = xrow & 15;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const u32x4 xlo = *reinterpret_cast<const u32x4*>(xr + (((8 * h + g) ^ sw) << 4));
    const u32x4 xhi = *reinterpret_cast<const u32x4*>(xr + (((8 * h + g + 4) ^ sw) << 4));
    const int xs = (int)((xs2[h] >> sshift) & 0xFFu);
#pragma unroll
    for (int i = 0; i < NS; ++i)
      acc[i] = mfma_scale_a8(wc[i][h], xlo, xhi, acc[i], (int)((sc2[i][h] >> sshift) & 0xFFu), xs);
  }
}

// The items of a workgroup, in three phases:
//   A  extra row groups (items it >= F, F = na * nquad, valid only for experts with more
//      than 16 rows; few), dealt round-robin, first, because each is as long as any other
//      item and leaving them to the end would lengthen the tail.  The extra group of item
//      j (the same expert and column quad as first-group item j) goes to workgroup
//      (j + XOFF) mod G, with XOFF = F mod G rounded up to a multiple of 8.  Round-robin
//      dealing leaves workgroups XOFF.. one first-group item short of the others (idle,
//      when F < G), so the extra groups even out the rounds instead of adding one; and
//      since workgroups are placed on the 8 XCDs round-robin, the extra group of item j
//      runs on the XCD of first-group item j, where the two reads of the same weight rows
//      can share that XCD's L2;
//   B  first-group items wg, wg + G, wg + 2G (STATIC_UNITS of them; G workgroups);
//   C  further first-group items: dealt round-robin too (StaticUnits), or claimed from a
//      device counter as workgroups become free (ClaimedUnits), so that workgroups that
//      stream faster, or drew lighter items, take more and all finish together.
// unit(n) gives the n-th phase-B/C item; enter(n) is called when the chunk loader, which
// reaches every item first, enters the n-th.
constexpr int STATIC_UNITS = 3;
struct StaticUnits {
  __device__ __forceinline__ int unit(int n) const { return (int)blockIdx.x + n * (int)gridDim.x; }
  __device__ __forceinline__ void enter(int) {}
};

// Claims: a launch with at most 5G first-group items claims nothing.  Otherwise workgroup
// w belongs to claim class j = w mod K (K = 16 classes, or G if fewer), and class j owns
// the dynamic items 3G + j, 3G + j + K, ...: its workgroups draw them in turn from the
// class's own counter.  Classes keep each counter's claims few (simultaneous claims on
// one word queue behind each other and slow every stream through its memory channel), and
// interleaving keeps their work alike.  No claim is issued at the start: the claim for the
// item at ordinal m + 2 is issued when the chunk loader enters ordinal m, and its result
// is written to the LDS queue when the loader enters ordinal m + 1, by which time it has
// long returned, so a claim never stalls the stream.  Claims are monotonic, so once a
// workgroup draws an item past the end every later claim of its class is past it too, and
// no item is lost.  `ctr` points at the class counters, CLAIM_STRIDE words apart; each
// class has an exit counter CLAIM_EXIT words after its claim counter (zero between
// launches; the class's last workgroup to finish resets both).
constexpr int DYNAMIC_MIN = 5;
static_assert(DYNAMIC_MIN >= STATIC_UNITS, "a dynamic launch has every static item");
constexpr int CLAIM_CLASSES = 16;
constexpr int CLAIM_STRIDE = 128;  // words between classes (512 bytes)
constexpr int CLAIM_EXIT = 32;     // exit counter, one 128-byte line after the claim counter
typedef __attribute__((address_space(3))) int32_t lds_i32;
struct ClaimedUnits {
  int32_t* ctr;
  lds_i32* q;      // 4 LDS words: claim results for ordinals n & 3
  int n_first;     // first-group items of the launch
  int pending;     // thread 0: the last claim issued
  bool claimed;    // thread 0: a claim was issued
  // Claiming pays once workgroups average more than DYNAMIC_MIN items; below that the
  // claims, issued in near lockstep, cost more than the balance gains.
  __device__ __forceinline__ bool dynamic() const { return n_first > DYNAMIC_MIN * (int)gridDim.x; }
  __device__ __forceinline__ int classes() const { return min(CLAIM_CLASSES, (int)gridDim.x); }
  __device__ __forceinline__ int cls() const { return (int)blockIdx.x % classes(); }
  __device__ __forceinline__ int32_t* class_ctr() const { return ctr + cls() * CLAIM_STRIDE; }
  // An increment-with-wrap (at 2^32 - 1: never reached) rather than an add: the compiler's
  // atomic optimizer turns a lone thread's add into a wave reduction that consumes the
  // result at once, which would stall the stream on every claim.
  __device__ __forceinline__ int claim() const {
    typedef __attribute__((address_space(1))) uint32_t global_u32;
    return (int)__builtin_amdgcn_atomic_inc32((volatile global_u32*)class_ctr(), 0xFFFFFFFFu, __ATOMIC_RELAXED,
                                              "agent");
  }
  __device__ __forceinline__ int unit(int n) const {
    // static launches deal every item round-robin: the 4th is past the end
    if (n < STATIC_UNITS || !dynamic()) return (int)blockIdx.x + n * (int)gridDim.x;
    return STATIC_UNITS * (int)gridDim.x + cls() + classes() * __builtin_amdgcn_readfirstlane(q[n & 3]);
  }
  // the chunk loader enters ordinal m (m >= 1): publish the claim for ordinal m + 1 (issued
  // when it entered ordinal m - 1), then claim for ordinal m + 2
  __device__ __forceinline__ void enter(int m) {
    if (threadIdx.x == 0 && dynamic()) {
      if (m + 1 >= STATIC_UNITS) q[(m + 1) & 3] = pending;
      if (m + 2 >= STATIC_UNITS) {
        pending = claim();
        claimed = true;
      }
    }
  }
  // After the workgroup's last item: its outstanding claim has been performed before the
  // exit count (its value is waited for), and the class's last workgroup resets the class.
  __device__ __forceinline__ void finish() {
    if (threadIdx.x == 0 && dynamic()) {
      if (claimed) {
        q[0] = pending;
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the claim has returned
      }
      const int K = classes();
      const int members = ((int)gridDim.x - 1 - cls()) / K + 1;
      int32_t* c = class_ctr();
      if (__hip_atomic_fetch_add(c + CLAIM_EXIT, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == members - 1) {
        __hip_atomic_store(c, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(c + CLAIM_EXIT, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
};

// Drive one workgroup over its items.  Policy P provides:
//   static constexpr int NS;   int nseg, n_items;   const uint16_t* xact;
//   int first_groups();   bool valid_lane(int it) (per lane);   ItemInfo info(int it);
//   u32x4 xload(const uint16_t*)                    -- one 16-byte activation load
//   void wait_inputs()                              -- before the first activation load
//   int x_row_offset(const ItemInfo&, int m)        -- element offset of activation row m
//   void w_setup(const ItemInfo&, int wave, WCursor<NS>&, int lane)   -- sets c.w
//   const uint8_t* scale_row(const ItemInfo&, int wave, int i, int r) -- scales of row r of subtile i
//   EpiState;  void c_setup(const ItemInfo&, int wave, EpiState&, int lane)
//   void epilogue(const EpiState&, const f32x4 (&acc)[NS], int lane)
//   static constexpr int XCHUNK;                    -- bytes of one activation chunk buffer
//   static constexpr bool ACT8;                     -- MXFP8 activations, scaled MFMA
//   typedef ScaleRun<...> Scales;                   -- scale staging run
// `xbufs` is 2 * P::XCHUNK bytes of LDS, `xctr` 2 zeroed LDS counters, `slab` this wave's
// SLAB_BYTES and `sslab` its P::Scales::slab_bytes<NS>() of LDS.  nseg must be a multiple of
// SPS and of the scale run (the launchers check it).
template <class P, int SPS, class Seq>
__device__ __forceinline__ void stream_items(P& p, Seq& seq, uint8_t* __restrict__ xbufs, uint32_t* xctr,
                                             uint8_t* __restrict__ slab, uint8_t* __restrict__ sslab, int wave,
                                             int lane) {
  constexpr int NS = P::NS;
  typedef typename P::Scales SR;
  constexpr int SL = SR::template loads<NS>();
  constexpr int XCHUNK_BYTES = P::XCHUNK;
  constexpr int XROUNDS = XGeom<XCHUNK_BYTES>::ROUNDS;
  static_assert(SR::SRUN % SPS == 0, "scale runs end on steps");
  const int tid = wave * 64 + lane;
  uint32_t lds_wr[2], lds_rd[2];
  for (int q = 0; q < 2; ++q) lds_wr[q] = slab_off((uint32_t)(lane >> 3) + 8u * q, (uint32_t)(lane & 7));
  for (int h = 0; h < 2; ++h) lds_rd[h] = slab_off((uint32_t)(lane & 15), (uint32_t)(lane >> 4) + 4u * h);
  const uint32_t sshift = 8u * (uint32_t)(lane >> 4);

  const int n_first = p.first_groups();
  const int wg = blockIdx.x, n_wg = gridDim.x;
  // phase A: the next valid extra-group item at or after `it` in this workgroup's stride.
  // Most candidates are invalid (only experts with more than 16 rows have extra groups),
  // and each check reads the active list and then the expert's count, so the candidates
  // are checked 64 at a time, one per lane: a scan costs two memory round trips per 64
  // candidates instead of two per candidate, and the first weight loads, which wait for
  // the scan, go out that much sooner.
  auto next_extra = [&](int it) {
    while (it < p.n_items) {
      const int c = it + lane * n_wg;
      const uint64_t ok = __ballot(c < p.n_items && p.valid_lane(c));
      if (ok) return it + (int)__builtin_ctzll(ok) * n_wg;
      it += 64 * n_wg;
    }
    return it;
  };
  // The next item after `c` (false past the end).  Only the chunk loader, which reaches
  // every item first, tells the sequence that a phase-B/C item is entered.
  auto pos_next = [&](const ItemPos& c, ItemPos& q, bool loader) {
    if (c.n < 0) {
      q.n = -1;
      q.it = next_extra(c.it + n_wg);
      if (q.it < p.n_items) return true;
    }
    q.n = c.n + 1;
    q.it = seq.unit(q.n);
    if (q.it >= n_first) return false;
    if (loader && q.n > 0) seq.enter(q.n);
    return true;
  };
  ItemPos first;
  first.n = -1;
  const int xoff = ((n_first % n_wg + 7) & ~7) % n_wg;  // XOFF
  first.it = next_extra(n_first + (wg + n_wg - xoff) % n_wg);
  if (first.it >= p.n_items) {
    first.n = 0;
    first.it = seq.unit(0);
    if (first.it >= n_first) return;
  }

  // ---- weight cursor (per wave): the step the ring is reloaded with.  Once the
  // workgroup's items are exhausted it stays on the last step (re-read, never used).
  WCursor<NS, SR> cw;
  auto cursor_setup = [&](const ItemPos& at) {
    const ItemInfo f = p.info(at.it);
    cw.at = at;
    cw.seg = 0;
    p.w_setup(f, wave, cw, lane);
#pragma unroll
    for (int k = 0; k < SL; ++k) {
      const int rho = (k * SR::ROWS_PER_LOAD + lane / SR::LANES_PER_ROW) % (NS * SUB_ROWS);
      cw.sr[k] = p.scale_row(f, wave, rho / SUB_ROWS, rho % SUB_ROWS) + (lane % SR::LANES_PER_ROW) * SR::LOAD;
    }
  };
  cursor_setup(first);
  auto advance_w = [&]() {
    if (cw.seg + SPS < p.nseg) {
      cw.seg += SPS;
    } else {
      ItemPos nx;
      if (pos_next(cw.at, nx, false)) cursor_setup(nx);
    }
  };
  WRing<NS, SPS> rw;
  typename SR::Reg sreg[SL];  // scales of the next run, loaded one step ahead

  // ---- activation chunks (per workgroup): the first one is loaded before the loop
  auto chunk_of = [&](const ItemPos& at, int c0) {
    XChunk ch;
    ch.at = at;
    ch.c0 = c0;
    ch.info = p.info(at.it);
    ch.ns = min(ch.info.cs, p.nseg - c0);
    return ch;
  };
  auto next_chunk = [&](const XChunk& ch, bool& ok) {
    ok = true;
    if (ch.c0 + ch.ns < p.nseg) return chunk_of(ch.at, ch.c0 + ch.ns);
    ItemPos nx;
    if (pos_next(ch.at, nx, true)) return chunk_of(nx, 0);
    ok = false;
    return ch;
  };
  // The first weight step and scale run are requested before anything else, so that the
  // first compute waits for one memory round trip, not for the chunk hand-off as well.
  wring_load(rw, cw);
  srun_load<NS, SR>(sreg, cw);
  p.wait_inputs();
  u32x4 xv[XROUNDS];
  XChunk cur = chunk_of(first, 0);
  xchunk_load(p, cur, xv, tid);
  xchunk_settle(p, cur, xv, tid);
  xchunk_put<XROUNDS, XCHUNK_BYTES, P::ACT8>(xbufs, cur, xv, tid);
  xready_publish(&xctr[0]);
  int xb = 0;                  // LDS buffer holding `cur`
  uint32_t gen[2] = {1u, 0u};  // chunks published so far into each buffer
  srun_store<NS, SR>(sslab, sreg, lane);
  advance_w();
  if (cw.seg % SR::SRUN == 0) srun_load<NS, SR>(sreg, cw);
  bool have_next;
  XChunk nxt = next_chunk(cur, have_next);
  if (have_next) xchunk_load(p, nxt, xv, tid);
  xready_wait(&xctr[0], WG_THREADS);

  // ---- compute cursor
  int cseg = 0;
  typename P::EpiState es;
  p.c_setup(cur.info, wave, es, lane);
  int xrow = ((lane & 15) < cur.info.rows) ? (lane & 15) : 0;

  f32x4 acc[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (;;) {
    // one step: SPS segments; each segment's ring slot is reloaded with the next step
#pragma unroll
    for (int jj = 0; jj < SPS; ++jj) {
      if constexpr (P::ACT8)
        segment_compute_a8<NS, SR, XCHUNK_BYTES>(rw.w[jj], sslab, (cseg + jj) % SR::SRUN, cw, cw.seg + jj,
                                                 xbufs + xb * XCHUNK_BYTES, cseg + jj - cur.c0, cur.info.rows, xrow,
                                                 slab, lds_wr, lds_rd, sshift, lane, acc);
      else
        segment_compute<NS, SR>(rw.w[jj], sslab, (cseg + jj) % SR::SRUN, cw, cw.seg + jj, xbufs + xb * XCHUNK_BYTES,
                                cseg + jj - cur.c0, cur.info.rows, xrow, slab, lds_wr, lds_rd, sshift, lane, acc);
    }
    advance_w();
    // Chunks and items end on step boundaries (their lengths are multiples of SPS).
    cseg += SPS;
    if (cseg >= cur.c0 + cur.ns) {
      // chunk done: publish this thread's pieces of the next chunk, wait for the rest
      if (have_next) {
        xchunk_settle(p, nxt, xv, tid);
        xchunk_put<XROUNDS, XCHUNK_BYTES, P::ACT8>(xbufs + (xb ^ 1) * XCHUNK_BYTES, nxt, xv, tid);
        xready_publish(&xctr[xb ^ 1]);
        gen[xb ^ 1] += 1u;
        xready_wait(&xctr[xb ^ 1], gen[xb ^ 1] * WG_THREADS);
      }
      if (cseg >= p.nseg) {
        p.epilogue(es, acc, lane);
#pragma unroll
        for (int i = 0; i < NS; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (!have_next) break;
        cseg = 0;
      }
      cur = nxt;
      xb ^= 1;
      if (cseg == 0) {
        p.c_setup(cur.info, wave, es, lane);
        xrow = ((lane & 15) < cur.info.rows) ? (lane & 15) : 0;
      }
      nxt = next_chunk(cur, have_next);
      if (have_next) xchunk_load(p, nxt, xv, tid);
    }
    // Scales: the next step starting a run finds its run in sreg (loaded when the weight
    // cursor reached it, one step ago); the wave's own earlier slab reads precede this
    // store in LDS order.  Then prefetch the run the cursor has just reached, if any.
    if (cseg % SR::SRUN == 0) srun_store<NS, SR>(sslab, sreg, lane);
    if (cw.seg % SR::SRUN == 0) srun_load<NS, SR>(sreg, cw);
  }
}

}  // namespace mx
