// Continuous weight streaming for the expert GEMMs (one workgroup = 4 wavefronts).
//
// Work items are (row group, expert, quad of column tiles); the 4 wavefronts of a
// workgroup take the 4 tiles of a quad, so they share one expert, one row group and one
// activation slice.  A workgroup owns a strided subset of the items and walks them
// back to back:
//
//   weights   each wave keeps its own register ring of DW steps; a step is SPS segments
//             (a segment = 256 K values of NS x 16 rows), requested back to back so each
//             row's SPS * 128 bytes hit one open DRAM page.  The ring runs across item
//             boundaries, so there is no pipeline drain between items.
//   acts      the activation rows of an item are staged in LDS, chunk by chunk, shared
//             by the 4 waves.  A chunk holds CS segments of the item's R rows, with
//             CS = 64 / R rounded down to a multiple of SPS (at least SPS), so a chunk is at
//             most 32 KB, is loaded by XROUNDS rounds of 16-byte loads of the 256 threads,
//             and ends on a step.  The loads of chunk i+1 are issued when chunk i starts and
//             written to the other LDS buffer when it ends; LDS counters hand it over.
//
// Vector memory instructions per wave and segment: 2 * NS weight loads, NS / 2 scale loads
// (16 bytes of one row = 2 segments) and on average 4 / CS activation loads; the MFMA
// activation operand is read from LDS.  Issuing activation loads per wave and segment,
// or one 8-byte scale load per row and segment, made the request count rather than the
// bytes the limit.
//
// Loads retire in issue order and every step issues the same weight loads (an exhausted
// cursor re-reads its last segment), so the compiler's waits stay exact: a step waits
// only for the segment it consumes.
#pragma once
#include "mx_device.hpp"

namespace mx {

constexpr int WG_WAVES = 4;
constexpr int XCHUNK_BYTES = 32768;  // one activation chunk: R rows x CS segments x 512 B
constexpr int XPIECES = XCHUNK_BYTES / 16;
constexpr int XROUNDS = XPIECES / (WG_WAVES * 64);

// One step of the weight ring: SPS consecutive segments of the wave's NS subtiles, so each
// row's SPS * 128 bytes are requested back to back (DRAM pages are opened once per step,
// not once per segment), plus their scales: 16 bytes per row cover two segments.
template <int NS, int SPS>
struct WRing {
  u32x4 w[SPS][NS][2];
  u32x4 s[NS][SPS / 2];
};

template <int NS>
struct WCursor {
  int it;   // current item
  int seg;  // first segment of the next step to load
  const uint8_t* w[NS][2];
  const uint8_t* s[NS];
};

template <int NS, int SPS>
__device__ __forceinline__ void wring_load(WRing<NS, SPS>& r, const WCursor<NS>& c) {
#pragma unroll
  for (int j = 0; j < SPS; ++j) {
    const size_t wo = (size_t)(c.seg + j) * SEG_BYTES;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      r.w[j][i][0] = ld_stream16(c.w[i][0] + wo);
      r.w[j][i][1] = ld_stream16(c.w[i][1] + wo);
    }
  }
#pragma unroll
  for (int i = 0; i < NS; ++i)
#pragma unroll
    for (int q = 0; q < SPS / 2; ++q) r.s[i][q] = ld16(c.s[i] + (size_t)(c.seg + 2 * q) * SEG_SCALES);
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
  int it;  // item
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

// Issue the activation loads of chunk `ch` (XROUNDS rounds of one 16-byte load per
// thread; threads past the chunk repeat its last piece).
template <class P>
__device__ __forceinline__ void xchunk_load(const P& p, const XChunk& ch, u32x4 (&xv)[XROUNDS], int tid) {
  const int R = ch.info.rows;
  const int npieces = R * ch.ns * 32;
  int rowoff[16];  // element offset of each row of the group (uniform)
#pragma unroll
  for (int m = 0; m < 16; ++m) rowoff[m] = (m < R) ? p.x_row_offset(ch.info, m) : 0;
#pragma unroll
  for (int r = 0; r < XROUNDS; ++r) {
    const int q = min(r * (WG_WAVES * 64) + tid, npieces - 1);
    const int rs = q >> 5, pc = q & 31;
    const int s = rs / R, m = rs - s * R;
    int ro = 0;
#pragma unroll
    for (int mm = 0; mm < 16; ++mm) ro = (m == mm) ? rowoff[mm] : ro;
    xv[r] = ld16(p.xact + (size_t)ro + (size_t)(ch.c0 + s) * SEG_K + pc * 8);
  }
}

__device__ __forceinline__ void xchunk_store(uint8_t* __restrict__ buf, const XChunk& ch, const u32x4 (&xv)[XROUNDS],
                                             int tid) {
  const int R = ch.info.rows;
  const int npieces = R * ch.ns * 32;
#pragma unroll
  for (int r = 0; r < XROUNDS; ++r) {
    const int q = min(r * (WG_WAVES * 64) + tid, npieces - 1);
    const int rs = q >> 5, pc = q & 31;
    const int s = rs / R, m = rs - s * R;
    *reinterpret_cast<u32x4*>(buf + xpiece_off(s, m, R, pc)) = xv[r];
  }
}

// Consume one segment: LDS transpose of the codes, decode, MFMA with activations from the
// chunk buffer (xrow: this lane's row within the chunk; rows past R read row 0, whose
// products land in output columns that are not stored).  sc2[i] holds the 8 scale bytes of
// subtile i's row (lane & 15) for this segment.
template <int NS>
__device__ __forceinline__ void segment_compute(const u32x4 (&w)[NS][2], const u32x2 (&sc2)[NS],
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
  const int j = lane >> 4;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float sc[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) sc[i] = e8m0_scale_operand((sc2[i][h] >> sshift) & 0xFFu);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bf16x8 xb =
          as_bf16x8(*reinterpret_cast<const u32x4*>(xbuf + xpiece_off(sl, xrow, R, (j + 4 * h) * 4 + c)));
#pragma unroll
      for (int i = 0; i < NS; ++i) acc[i] = mfma_bf16(decode8(wc[i][h][c], sc[i]), xb, acc[i]);
    }
  }
}

// Drive one workgroup over its items.  Policy P provides:
//   static constexpr int NS;   int nseg, n_items;   const uint16_t* xact;
//   bool valid(int it);   ItemInfo info(int it);
//   int x_row_offset(const ItemInfo&, int m)        -- element offset of activation row m
//   void w_setup(const ItemInfo&, int wave, WCursor<NS>&, int lane)
//   EpiState;  void c_setup(const ItemInfo&, int wave, EpiState&, int lane)
//   void epilogue(const EpiState&, const f32x4 (&acc)[NS], int lane)
// `xbufs` is 2 * XCHUNK_BYTES of LDS, `xctr` 2 zeroed LDS counters, `slab` this wave's
// SLAB_BYTES of LDS.
template <class P, int SPS, int DW>
__device__ __forceinline__ void stream_items(P& p, uint8_t* __restrict__ xbufs, uint32_t* xctr,
                                             uint8_t* __restrict__ slab, int wave, int lane) {
  constexpr int NS = P::NS;
  const int tid = wave * 64 + lane;
  const int wg = blockIdx.x, n_wg = gridDim.x;
  uint32_t lds_wr[2], lds_rd[2];
  for (int q = 0; q < 2; ++q) lds_wr[q] = slab_off((uint32_t)(lane >> 3) + 8u * q, (uint32_t)(lane & 7));
  for (int h = 0; h < 2; ++h) lds_rd[h] = slab_off((uint32_t)(lane & 15), (uint32_t)(lane >> 4) + 4u * h);
  const uint32_t sshift = 8u * (uint32_t)(lane >> 4);

  auto next_valid = [&](int it) {
    while (it < p.n_items && !p.valid(it)) it += n_wg;
    return it;
  };
  const int first = next_valid(wg);
  if (first >= p.n_items) return;

  // ---- weight cursor (per wave) and its ring
  WCursor<NS> cw;
  cw.it = first;
  cw.seg = 0;
  p.w_setup(p.info(first), wave, cw, lane);
  auto advance_w = [&]() {
    if (cw.seg + SPS < p.nseg) {
      cw.seg += SPS;
    } else {
      const int nx = next_valid(cw.it + n_wg);
      if (nx < p.n_items) {
        cw.it = nx;
        cw.seg = 0;
        p.w_setup(p.info(nx), wave, cw, lane);
      }
    }
  };
  WRing<NS, SPS> rw[DW];

  // ---- activation chunks (per workgroup): the first one is loaded before the loop
  auto chunk_of = [&](int it, int c0) {
    XChunk ch;
    ch.it = it;
    ch.c0 = c0;
    ch.info = p.info(it);
    ch.ns = min(ch.info.cs, p.nseg - c0);
    return ch;
  };
  auto next_chunk = [&](const XChunk& ch, bool& ok) {
    ok = true;
    if (ch.c0 + ch.ns < p.nseg) return chunk_of(ch.it, ch.c0 + ch.ns);
    const int nx = next_valid(ch.it + n_wg);
    if (nx < p.n_items) return chunk_of(nx, 0);
    ok = false;
    return ch;
  };
  u32x4 xv[XROUNDS];
  XChunk cur = chunk_of(first, 0);
  xchunk_load(p, cur, xv, tid);
  xchunk_store(xbufs, cur, xv, tid);
  xready_publish(&xctr[0]);
  int xb = 0;          // LDS buffer holding `cur`
  uint32_t gen[2] = {1u, 0u};  // chunks published so far into each buffer
  xready_wait(&xctr[0], WG_THREADS);
  bool have_next;
  XChunk nxt = next_chunk(cur, have_next);
  if (have_next) xchunk_load(p, nxt, xv, tid);
  // The weight ring is filled after the next chunk's activation loads, so on every path
  // into the loop at least DW steps of weight loads follow them and the wait before
  // their LDS store never drains the weight stream.
#pragma unroll
  for (int d = 0; d < DW; ++d) {
    wring_load(rw[d], cw);
    advance_w();
  }

  // ---- compute cursor
  int cit = first, cseg = 0;
  typename P::EpiState es;
  p.c_setup(cur.info, wave, es, lane);
  int xrow = ((lane & 15) < cur.info.rows) ? (lane & 15) : 0;

  f32x4 acc[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  while (cit < p.n_items) {
#pragma unroll
    for (int u = 0; u < DW; ++u) {
      if (cit < p.n_items) {
#pragma unroll
        for (int jj = 0; jj < SPS; ++jj) {
          u32x2 sc2[NS];
#pragma unroll
          for (int i = 0; i < NS; ++i) {
            const u32x4 q = rw[u].s[i][jj / 2];
            sc2[i] = (jj & 1) ? u32x2{q[2], q[3]} : u32x2{q[0], q[1]};
          }
          segment_compute<NS>(rw[u].w[jj], sc2, xbufs + xb * XCHUNK_BYTES, cseg + jj - cur.c0, cur.info.rows, xrow,
                              slab, lds_wr, lds_rd, sshift, lane, acc);
        }
        // Chunks and items end on step boundaries (their lengths are multiples of SPS), so
        // this bookkeeping runs between steps, after which the next weight loads follow.
        cseg += SPS;
        if (cseg >= cur.c0 + cur.ns) {
          // chunk done: publish this thread's pieces of the next chunk, wait for the rest
          if (have_next) {
            xchunk_store(xbufs + (xb ^ 1) * XCHUNK_BYTES, nxt, xv, tid);
            xready_publish(&xctr[xb ^ 1]);
            gen[xb ^ 1] += 1u;
            xready_wait(&xctr[xb ^ 1], gen[xb ^ 1] * WG_THREADS);
          }
          if (cseg >= p.nseg) {
            p.epilogue(es, acc, lane);
#pragma unroll
            for (int i = 0; i < NS; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            cit = have_next ? nxt.it : p.n_items;
            cseg = 0;
          }
          if (have_next) {
            cur = nxt;
            xb ^= 1;
            if (cseg == 0) {
              p.c_setup(cur.info, wave, es, lane);
              xrow = ((lane & 15) < cur.info.rows) ? (lane & 15) : 0;
            }
            nxt = next_chunk(cur, have_next);
            if (have_next) xchunk_load(p, nxt, xv, tid);
          }
        }
      }
      wring_load(rw[u], cw);
      advance_w();
    }
  }
}

}  // namespace mx
