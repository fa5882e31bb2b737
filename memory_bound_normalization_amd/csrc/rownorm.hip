// Row-wise norms for gfx950 with each row staged in LDS: RMSNorm, residual add
// + RMSNorm, LayerNorm and L2Norm, on bf16 or fp16 data (fp16 is among the
// broadened inputs of "[Inductor] Codegen Gluon", section 3.2). RMSNorm rows
// of exactly 32768 and 65536 elements, and small launches (up to a few
// thousand rows) at exactly 2048, 4096, 8192 and 16384 for the widths and
// norms the launch tables list, are held in VGPRs instead
// (rownorm_regs_kernel, below).
//
// The method ("[Inductor] Codegen Gluon", section 3.1, RMSNorm as the reference
// workload; section 3.2 for the rest of the family): the input row is needed
// by the reduction and again by the normalize pass, so each row is read from
// HBM once into on-chip memory, kept narrow (bf16) there, and widened to fp32
// only where it is computed on. On gfx950 the row copy is a burst of
// global_load_lds_dwordx4 (HBM -> LDS without passing through VGPRs), issued
// for the whole row before the first wait, so a workgroup keeps its entire row
// in flight. The first pass either waits for the whole row set or, in the
// kernels the launch tables ask for it (large grids), takes each chunk as it
// lands: loads complete in issue order, so s_waitcnt on the number of copies
// still outstanding marks each chunk's arrival.
//
// Work decomposition: a workgroup holds ROWS row slots; each row is served by
// WPR waves (64 * WPR lanes). Lane t of a row owns the 16-byte chunks
// k = j * (64 * WPR) + t, j < MAXC, and reads back only the chunks it loaded,
// so the LDS passes need no barrier; the only barriers are the cross-wave
// steps of the reductions. Those need one float per wave of LDS; rather than
// allocate it beside the row (LDS is allocated in coarse granules, and 16
// extra bytes on a 32 KiB row would cost one resident workgroup per CU), each
// lane keeps its first chunk in VGPRs after the first pass and the wave parks
// its partial sums in that chunk's LDS slot, which nothing reads afterwards.
// The LDS footprint is exactly ROWS * N * 2 bytes.
//
// Modes (compile time):
//   kRms     y = x * rstd * w,            rstd = 1/sqrt(mean(x^2) + eps)
//   kAddRms  h = bf16(x + r) is stored, and replaces x in the LDS row;
//            y = h * rstd(h) * w          (r is read into VGPRs, used once)
//   kLayer   y = (x - mu) * rstd * w + b, mu = mean(x), rstd = 1/sqrt(var + eps),
//            var = mean((x - mu)^2): a second reduction over the staged row
//   kL2      y = x / max(||x||_2, eps)
#include "device.h"
#include "kernels.h"

// Timeline marks of the one-shot kernel: workgroup start, rows landed and
// reduced, last store issued and completed. The measurement tools compile this
// file with them defined (wall clock per workgroup); in the library they are
// empty and the kernel is unchanged.
#ifndef MBN_TL_START
#define MBN_TL_START()
#define MBN_TL_LANDED()
#define MBN_TL_END()
#endif

namespace mbn {
namespace {

// Sums of v[rr] over the WPR waves of each of the RPL rows a lane set serves,
// with one barrier for all of them. The wave totals go to `part` when given
// (a small LDS array, [2][RPL][WPR] floats: `which` selects the half), else
// they are parked in float `which` of each wave's first chunk of that row
// (see the header comment).
template <int WPR, int RPL>
__device__ __forceinline__ void rows_sum(float (&v)[RPL], u32x4* buf0, float* part, int nchunk,
                                         int t, int wave, int which) {
#pragma unroll
  for (int rr = 0; rr < RPL; ++rr) v[rr] = wave_sum(v[rr]);
  if constexpr (WPR > 1) {
    if ((t & 63) == 0) {
#pragma unroll
      for (int rr = 0; rr < RPL; ++rr) {
        if (part) part[(which * RPL + rr) * WPR + wave] = v[rr];
        else reinterpret_cast<float*>(buf0 + (size_t)rr * nchunk)[wave * 256 + which] = v[rr];  // 256 floats = 64 chunks
      }
    }
    __syncthreads();
#pragma unroll
    for (int rr = 0; rr < RPL; ++rr) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < WPR; ++i)
        s += part ? part[(which * RPL + rr) * WPR + i]
                  : reinterpret_cast<const float*>(buf0 + (size_t)rr * nchunk)[i * 256 + which];
      v[rr] = s;
    }
  }
}

// HBM -> LDS for the RPL rows starting at row0: every chunk in flight before
// any wait. Lane t of the lane set loads chunks j * 64 * WPR + t.
template <int WPR, int RPL, int MAXC, bool FULL>
__device__ __forceinline__ void stage_rows(const RowNormArgs& a, u32x4* buf0, int64_t row0, int t,
                                           int wave) {
  constexpr int TPR = 64 * WPR;
  const int nchunk = a.nchunk;
#pragma unroll
  for (int rr = 0; rr < RPL; ++rr) {
    if (row0 + rr < a.M) {
      const u32x4* xrow = reinterpret_cast<const u32x4*>(a.x) + (row0 + rr) * nchunk;
      u32x4* buf = buf0 + (size_t)rr * nchunk;
#pragma unroll
      for (int j = 0; j < MAXC; ++j) {
        const int k = j * TPR + t;
        if (FULL || k < nchunk) load_lds_16(xrow + k, (lds_void*)(buf + j * TPR + wave * 64));
      }
    }
  }
}

template <Norm MODE>
struct Regs {
  static constexpr bool kHasW = MODE != Norm::kL2;
  static constexpr bool kHasB = MODE == Norm::kLayer;
  static constexpr bool kHasR = MODE == Norm::kAddRms;
};

// Weight (and bias) chunks of this lane into VGPRs: L2 hits after the first rows.
template <Norm MODE, int WPR, int MAXC, bool FULL>
__device__ __forceinline__ void load_affine(const RowNormArgs& a, int t,
                                            u32x4 (&wreg)[Regs<MODE>::kHasW ? MAXC : 1],
                                            u32x4 (&breg)[Regs<MODE>::kHasB ? MAXC : 1]) {
  constexpr int TPR = 64 * WPR;
#pragma unroll
  for (int j = 0; j < MAXC; ++j) {
    const int k = j * TPR + t;
    const bool in = FULL || k < a.nchunk;
    if constexpr (Regs<MODE>::kHasW)
      wreg[j] = in ? reinterpret_cast<const u32x4*>(a.w)[k] : u32x4{0u, 0u, 0u, 0u};
    if constexpr (Regs<MODE>::kHasB)
      breg[j] = in ? reinterpret_cast<const u32x4*>(a.b)[k] : u32x4{0u, 0u, 0u, 0u};
  }
}

// The passes of the persistent kernel, once a row set has landed in LDS:
// pass 1 (sum of squares, or sum for LayerNorm), the reductions (LayerNorm: a
// second, centred pass), and pass 2 (normalize, weight, round, streaming
// stores). The same arithmetic, in the same order, as the one-shot kernel.
template <Norm MODE, typename DT, int WPR, int RPL, int MAXC, bool FULL>
__device__ __forceinline__ void finish_rows(const RowNormArgs& a, u32x4* buf0, float* part,
                                            int64_t row0, int t, int wave,
                                            const u32x4 (&wreg)[Regs<MODE>::kHasW ? MAXC : 1],
                                            const u32x4 (&breg)[Regs<MODE>::kHasB ? MAXC : 1]) {
  static_assert(!Regs<MODE>::kHasR, "the residual add runs one-shot only");
  constexpr int TPR = 64 * WPR;
  const int nchunk = a.nchunk;
  float s1[RPL];
  u32x4 first[RPL];  // chunk j = 0 of each row, kept for the later passes
#pragma unroll
  for (int rr = 0; rr < RPL; ++rr) {
    const u32x4* buf = buf0 + (size_t)rr * nchunk;
    float acc0 = 0.f, acc1 = 0.f;
    first[rr] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < MAXC; ++j) {
      const int k = j * TPR + t;
      if (FULL || k < nchunk) {
        const u32x4 v = buf[k];
        if (j == 0) first[rr] = v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = DT::lo(v[e]);
          const float q = DT::hi(v[e]);
          if constexpr (MODE == Norm::kLayer) {
            acc0 += p;
            acc1 += q;
          } else {
            acc0 = __builtin_fmaf(p, p, acc0);
            acc1 = __builtin_fmaf(q, q, acc1);
          }
        }
      }
    }
    s1[rr] = acc0 + acc1;
  }
  rows_sum<WPR, RPL>(s1, buf0, part, nchunk, t, wave, 0);

  float mu[RPL], scale[RPL];
  if constexpr (MODE == Norm::kLayer) {
    // Pass 1b (from LDS): centred second moment.
    float s2[RPL];
#pragma unroll
    for (int rr = 0; rr < RPL; ++rr) {
      const u32x4* buf = buf0 + (size_t)rr * nchunk;
      mu[rr] = s1[rr] * a.inv_n;
      float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
      for (int j = 0; j < MAXC; ++j) {
        const int k = j * TPR + t;
        if (FULL || k < nchunk) {
          const u32x4 v = (j == 0) ? first[rr] : buf[k];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p = DT::lo(v[e]) - mu[rr];
            const float q = DT::hi(v[e]) - mu[rr];
            acc0 = __builtin_fmaf(p, p, acc0);
            acc1 = __builtin_fmaf(q, q, acc1);
          }
        }
      }
      s2[rr] = acc0 + acc1;
    }
    rows_sum<WPR, RPL>(s2, buf0, part, nchunk, t, wave, 1);
#pragma unroll
    for (int rr = 0; rr < RPL; ++rr) scale[rr] = __builtin_amdgcn_rsqf(s2[rr] * a.inv_n + a.eps);
  } else if constexpr (MODE == Norm::kL2) {
#pragma unroll
    for (int rr = 0; rr < RPL; ++rr) {
      const float nrm = __builtin_sqrtf(s1[rr]);
      scale[rr] = 1.0f / ((nrm < a.eps) ? a.eps : nrm);  // NaN norms stay NaN
      mu[rr] = 0.f;
    }
  } else {
#pragma unroll
    for (int rr = 0; rr < RPL; ++rr) {
      scale[rr] = __builtin_amdgcn_rsqf(__builtin_fmaf(s1[rr], a.inv_n, a.eps));
      mu[rr] = 0.f;
    }
  }

  // Pass 2 (from LDS): normalize, weight, round, streaming stores.
#pragma unroll
  for (int rr = 0; rr < RPL; ++rr) {
    if (row0 + rr >= a.M) continue;
    const u32x4* buf = buf0 + (size_t)rr * nchunk;
    u32x4* yrow = reinterpret_cast<u32x4*>(a.y) + (row0 + rr) * nchunk;
#pragma unroll
    for (int j = 0; j < MAXC; ++j) {
      const int k = j * TPR + t;
      if (FULL || k < nchunk) {
        const u32x4 v = (j == 0) ? first[rr] : buf[k];
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float p = DT::lo(v[e]), q = DT::hi(v[e]);
          if constexpr (MODE == Norm::kLayer) {
            p = __builtin_fmaf((p - mu[rr]) * scale[rr], DT::lo(wreg[j][e]), DT::lo(breg[j][e]));
            q = __builtin_fmaf((q - mu[rr]) * scale[rr], DT::hi(wreg[j][e]), DT::hi(breg[j][e]));
          } else if constexpr (MODE == Norm::kL2) {
            p *= scale[rr];
            q *= scale[rr];
          } else {
            p = (p * scale[rr]) * DT::lo(wreg[j][e]);
            q = (q * scale[rr]) * DT::hi(wreg[j][e]);
          }
          o[e] = DT::pack(p, q);
        }
        store_nt_16(yrow + k, o);
      }
    }
  }
}

// One-shot kernel: one workgroup = ROWS lane sets of 64 * WPR lanes; each
// lane set serves RPL consecutive rows with the same lanes, so one set of
// weight (and bias) registers serves RPL rows and the weight is fetched from
// L2 once per RPL rows. FULL: the row is exactly MAXC chunks per lane (the
// power-of-two widths), so no chunk needs a bounds predicate.
//
// Its staging and passes stay in this one body rather than calling the
// helpers above: with the row copy issued from a separate inlined helper the
// compiler scheduled the LDS reads of the LayerNorm passes less far ahead,
// 4-6% slower at N >= 16384 on MI355X (RMSNorm, L2Norm and the residual add
// unchanged).
//
// rownorm_block is that body for one row block (ROWS * RPL rows starting at
// block * ROWS * RPL); rownorm_kernel runs it for its own block. LATE_W
// (rownorm_lw_kernel) loads the weight (and bias) only once the row is
// reduced, just before pass 2, instead of alongside the row copy: on MI355X
// the weight loads issued with the copy slowed the 512-lane, one-row
// workgroups of the N <= 8192 band by 3-8% (L2Norm, which reads no weight,
// ran that much faster on the same geometry), while waiting for them after
// the reduction costs less. Not with per-chunk waits, whose kernels load the
// weight first: there a weight loaded after the reduction measured 3-11%
// slower at N = 16384 (4096 ... 16384 rows).
template <Norm MODE, typename DT, int WPR, int ROWS, int RPL, int MAXC, bool FULL, bool CHUNK_WAIT,
          bool LATE_W = false>
__device__ __forceinline__ void rownorm_block(const RowNormArgs& a, int64_t block) {
  constexpr int TPR = 64 * WPR;  // lanes per lane set
  constexpr bool kHasW = MODE != Norm::kL2;
  constexpr bool kHasB = MODE == Norm::kLayer;
  constexpr bool kHasR = MODE == Norm::kAddRms;
  // Pass 1 consumes each staged chunk as it lands (see below): full-width
  // kernels of the table entries that ask for it, not the residual add.
  constexpr bool kChunkWait = CHUNK_WAIT && FULL && !kHasR;
  static_assert(!(LATE_W && CHUNK_WAIT), "late weights are for kernels without per-chunk waits");
  extern __shared__ u32x4 lds_rows[];  // ROWS * RPL * nchunk chunks (or more, see launcher)
  MBN_TL_START();

  const int nchunk = a.nchunk;
  const int tid = threadIdx.x;
  const int slot = tid / TPR;
  const int t = tid - slot * TPR;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t row0 = (block * ROWS + slot) * RPL;

  u32x4* buf0 = lds_rows + (size_t)slot * RPL * nchunk;  // row rr at buf0 + rr * nchunk

  u32x4 rreg[kHasR ? RPL : 1][kHasR ? MAXC : 1], wreg[kHasW ? MAXC : 1], breg[kHasB ? MAXC : 1];
  float s1[RPL];
  u32x4 first[RPL];  // chunk j = 0 of each row, kept for the later passes
  if constexpr (kChunkWait) {
    // Weights and bias go to VGPRs (L2 hits after the first rows). With
    // per-chunk waits they are loaded before the row copy, so that every
    // vector-memory load issued after a row chunk's copy is a later chunk's copy.
#pragma unroll
    for (int j = 0; j < MAXC; ++j) {
      const int k = j * TPR + t;
      if constexpr (kHasW) wreg[j] = reinterpret_cast<const u32x4*>(a.w)[k];
      if constexpr (kHasB) breg[j] = reinterpret_cast<const u32x4*>(a.b)[k];
    }
    // The per-chunk waits below count the copies issued after chunk q. Their
    // immediates assume the weight / bias loads were all issued before the
    // first copy: a weight load sunk below a copy would make the wait for an
    // earlier chunk also wait for it (correct, but it puts an L2 round trip
    // back on pass 1's path), and nothing else keeps them apart (the loads
    // read global memory, the copies write LDS). The empty asm with a memory
    // clobber keeps the IR order, the scheduling barrier keeps the machine
    // scheduler from interleaving the two groups. Correctness rests on the
    // copies themselves staying in program order (each writes LDS through
    // M0; the compiler keeps them in order), so that exactly the later copies
    // are outstanding after chunk q's.
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int rr = 0; rr < RPL; ++rr) {
      if (row0 + rr < a.M) {
        const u32x4* xrow = reinterpret_cast<const u32x4*>(a.x) + (row0 + rr) * nchunk;
        u32x4* buf = buf0 + (size_t)rr * nchunk;
#pragma unroll
        for (int j = 0; j < MAXC; ++j) load_lds_16(xrow + j * TPR + t, (lds_void*)(buf + j * TPR + wave * 64));
      }
    }
    // Pass 1 (from LDS): sum of squares, or sum for LayerNorm, one chunk at a
    // time. Vector-memory loads complete in issue order, and with every row of
    // the lane set copied (no row past M) the RPL * MAXC copies were issued last,
    // so copy q (row q / MAXC, chunk q % MAXC) has landed once at most
    // RPL * MAXC - 1 - q loads are outstanding: each chunk is taken as it lands
    // instead of after the whole row set, in the same order and with the same
    // arithmetic. In the grid's last row sets it waits for every load.
    float acc0[RPL], acc1[RPL];
#pragma unroll
    for (int rr = 0; rr < RPL; ++rr) {
      acc0[rr] = 0.f;
      acc1[rr] = 0.f;
    }
    auto take = [&](int rr, int j) {
      const u32x4 v = buf0[(size_t)rr * nchunk + j * TPR + t];
      if (j == 0) first[rr] = v;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = DT::lo(v[e]);
        const float q = DT::hi(v[e]);
        if constexpr (MODE == Norm::kLayer) {
          acc0[rr] += p;
          acc1[rr] += q;
        } else {
          acc0[rr] = __builtin_fmaf(p, p, acc0[rr]);
          acc1[rr] = __builtin_fmaf(q, q, acc1[rr]);
        }
      }
    };
    if (row0 + RPL <= a.M) {
      static_for<0, RPL * MAXC>([&](auto q) {
        constexpr int Q = decltype(q)::value;
        wait_vmcnt_le<RPL * MAXC - 1 - Q>();
        take(Q / MAXC, Q % MAXC);
      });
    } else {
      wait_vmem();
#pragma unroll
      for (int rr = 0; rr < RPL; ++rr)
#pragma unroll
        for (int j = 0; j < MAXC; ++j) take(rr, j);
    }
#pragma unroll
    for (int rr = 0; rr < RPL; ++rr) s1[rr] = acc0[rr] + acc1[rr];
  } else {
    // HBM -> LDS: every row of the lane set, all chunks in flight before any wait.
#pragma unroll
    for (int rr = 0; rr < RPL; ++rr) {
      if (row0 + rr < a.M) {
        const u32x4* xrow = reinterpret_cast<const u32x4*>(a.x) + (row0 + rr) * nchunk;
        u32x4* buf = buf0 + (size_t)rr * nchunk;
#pragma unroll
        for (int j = 0; j < MAXC; ++j) {
          const int k = j * TPR + t;
          if (FULL || k < nchunk) load_lds_16(xrow + k, (lds_void*)(buf + j * TPR + wave * 64));
        }
      }
    }
    // Residual chunks go to VGPRs (consumed once); weights and bias to VGPRs
    // (L2 hits after the first rows), all overlapping the row copy.
#pragma unroll
    for (int j = 0; j < MAXC; ++j) {
      const int k = j * TPR + t;
      const bool in = FULL || k < nchunk;
      if constexpr (kHasR) {
#pragma unroll
        for (int rr = 0; rr < RPL; ++rr)
          rreg[rr][j] = (row0 + rr < a.M && in)
                            ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.r) + (row0 + rr) * nchunk + k)
                            : u32x4{0u, 0u, 0u, 0u};
      }
      if constexpr (kHasW && !LATE_W) wreg[j] = in ? reinterpret_cast<const u32x4*>(a.w)[k] : u32x4{0u, 0u, 0u, 0u};
      if constexpr (kHasB && !LATE_W) breg[j] = in ? reinterpret_cast<const u32x4*>(a.b)[k] : u32x4{0u, 0u, 0u, 0u};
    }
    wait_vmem();

    // Pass 1 (from LDS): sum of squares, or sum for LayerNorm. For the residual
    // add, h = bf16(x + r) is formed here, written back over x in LDS and
    // stored; the norm is taken of the rounded h.
#pragma unroll
    for (int rr = 0; rr < RPL; ++rr) {
      u32x4* buf = buf0 + (size_t)rr * nchunk;
      const bool live = row0 + rr < a.M;
      float acc0 = 0.f, acc1 = 0.f;
      first[rr] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < MAXC; ++j) {
        const int k = j * TPR + t;
        if (FULL || k < nchunk) {
          u32x4 v = buf[k];
          if constexpr (kHasR) {
            u32x4 hv;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              hv[e] = DT::pack(DT::lo(v[e]) + DT::lo(rreg[rr][j][e]),
                                  DT::hi(v[e]) + DT::hi(rreg[rr][j][e]));
            v = hv;
            buf[k] = hv;
            if (live) store_nt_16(reinterpret_cast<u32x4*>(a.h) + (row0 + rr) * nchunk + k, hv);
          }
          if (j == 0) first[rr] = v;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p = DT::lo(v[e]);
            const float q = DT::hi(v[e]);
            if constexpr (MODE == Norm::kLayer) {
              acc0 += p;
              acc1 += q;
            } else {
              acc0 = __builtin_fmaf(p, p, acc0);
              acc1 = __builtin_fmaf(q, q, acc1);
            }
          }
        }
      }
      s1[rr] = acc0 + acc1;
    }
  }
  // Chunk wave * 64 of each row (lane 0's first chunk) is in VGPRs now and is
  // not read from LDS again; the launch tables guarantee nchunk >= 64 * WPR, so
  // every wave owns such a chunk to park its partial sums in.
  rows_sum<WPR, RPL>(s1, buf0, nullptr, nchunk, t, wave, 0);
  MBN_TL_LANDED();

  float mu[RPL], scale[RPL];
  if constexpr (MODE == Norm::kLayer) {
    // Pass 1b (from LDS): centred second moment.
    float s2[RPL];
#pragma unroll
    for (int rr = 0; rr < RPL; ++rr) {
      const u32x4* buf = buf0 + (size_t)rr * nchunk;
      mu[rr] = s1[rr] * a.inv_n;
      float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
      for (int j = 0; j < MAXC; ++j) {
        const int k = j * TPR + t;
        if (FULL || k < nchunk) {
          const u32x4 v = (j == 0) ? first[rr] : buf[k];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p = DT::lo(v[e]) - mu[rr];
            const float q = DT::hi(v[e]) - mu[rr];
            acc0 = __builtin_fmaf(p, p, acc0);
            acc1 = __builtin_fmaf(q, q, acc1);
          }
        }
      }
      s2[rr] = acc0 + acc1;
    }
    rows_sum<WPR, RPL>(s2, buf0, nullptr, nchunk, t, wave, 1);
#pragma unroll
    for (int rr = 0; rr < RPL; ++rr) scale[rr] = __builtin_amdgcn_rsqf(s2[rr] * a.inv_n + a.eps);
  } else if constexpr (MODE == Norm::kL2) {
#pragma unroll
    for (int rr = 0; rr < RPL; ++rr) {
      const float nrm = __builtin_sqrtf(s1[rr]);
      scale[rr] = 1.0f / ((nrm < a.eps) ? a.eps : nrm);  // NaN norms stay NaN
      mu[rr] = 0.f;
    }
  } else {
#pragma unroll
    for (int rr = 0; rr < RPL; ++rr) {
      scale[rr] = __builtin_amdgcn_rsqf(__builtin_fmaf(s1[rr], a.inv_n, a.eps));
      mu[rr] = 0.f;
    }
  }

  if constexpr (LATE_W) load_affine<MODE, WPR, MAXC, FULL>(a, t, wreg, breg);

  // Pass 2 (from LDS): normalize, weight, round to bf16, streaming stores.
#pragma unroll
  for (int rr = 0; rr < RPL; ++rr) {
    if (row0 + rr >= a.M) continue;
    const u32x4* buf = buf0 + (size_t)rr * nchunk;
    u32x4* yrow = reinterpret_cast<u32x4*>(a.y) + (row0 + rr) * nchunk;
#pragma unroll
    for (int j = 0; j < MAXC; ++j) {
      const int k = j * TPR + t;
      if (FULL || k < nchunk) {
        const u32x4 v = (j == 0) ? first[rr] : buf[k];
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float p = DT::lo(v[e]), q = DT::hi(v[e]);
          if constexpr (MODE == Norm::kLayer) {
            p = __builtin_fmaf((p - mu[rr]) * scale[rr], DT::lo(wreg[j][e]), DT::lo(breg[j][e]));
            q = __builtin_fmaf((q - mu[rr]) * scale[rr], DT::hi(wreg[j][e]), DT::hi(breg[j][e]));
          } else if constexpr (MODE == Norm::kL2) {
            p *= scale[rr];
            q *= scale[rr];
          } else {
            p = (p * scale[rr]) * DT::lo(wreg[j][e]);
            q = (q * scale[rr]) * DT::hi(wreg[j][e]);
          }
          o[e] = DT::pack(p, q);
        }
        store_nt_16(yrow + k, o);
      }
    }
  }
  MBN_TL_END();
}

template <Norm MODE, typename DT, int WPR, int ROWS, int RPL, int MAXC, bool FULL, bool CHUNK_WAIT = false>
__global__ void __launch_bounds__(64 * WPR * ROWS) rownorm_kernel(RowNormArgs a) {
  rownorm_block<MODE, DT, WPR, ROWS, RPL, MAXC, FULL, CHUNK_WAIT>(a, xcd_remap(blockIdx.x, gridDim.x, a.xcd_group));
}

// The same one-shot kernel with the weight (and bias) loaded after the
// reduction (rownorm_block's LATE_W).
template <Norm MODE, typename DT, int WPR, int ROWS, int RPL, int MAXC, bool FULL>
__global__ void __launch_bounds__(64 * WPR * ROWS) rownorm_lw_kernel(RowNormArgs a) {
  rownorm_block<MODE, DT, WPR, ROWS, RPL, MAXC, FULL, false, true>(a, xcd_remap(blockIdx.x, gridDim.x, a.xcd_group));
}

// Register-resident rows: the same one-shot method with each lane's chunks of
// the row held in VGPRs instead of LDS ("[Inductor] Codegen Gluon", sections 2
// and 3.1 keep the reused row in on-chip memory; here that memory is the
// register file). Each row is still read from HBM once, with the same 16-byte
// non-temporal loads and the same lane-to-chunk mapping, kept narrow (packed
// 16-bit) in the registers and widened where it is computed on; both passes
// read those registers, so only the cross-wave partial sums use LDS (a small
// static array). The compiler's waits take each chunk as it lands (loads
// complete in issue order). The launch tables use it for the widths where it
// measured faster on MI355X: no LDS staging means no LDS write and two fewer
// LDS reads per chunk on each workgroup's critical path, at the same number of
// rows in flight (waves or VGPRs, not LDS, bound the residency there).
// Arithmetic, order and rounding are those of rownorm_block, so a row gives
// the same output bits through either kernel at the same WPR.
template <Norm MODE, typename DT, int WPR, int ROWS, int MAXC, bool FULL>
__global__ void __launch_bounds__(64 * WPR * ROWS) rownorm_regs_kernel(RowNormArgs a) {
  constexpr int TPR = 64 * WPR;  // lanes per row
  constexpr bool kHasW = Regs<MODE>::kHasW;
  constexpr bool kHasB = Regs<MODE>::kHasB;
  constexpr bool kHasR = Regs<MODE>::kHasR;
  __shared__ float part[ROWS][2][WPR];  // [row slot][reduction][wave]

  const int nchunk = a.nchunk;
  const int slot = __builtin_amdgcn_readfirstlane(threadIdx.x / TPR);  // TPR is whole waves
  const int t = threadIdx.x - slot * TPR;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t row = xcd_remap(blockIdx.x, gridDim.x, a.xcd_group) * ROWS + slot;
  const bool live = row < a.M;
  // With one row per workgroup, a workgroup past the last row has no barrier
  // to join: it leaves here, and the row loads below need no row predicate
  // (on MI355X predicated loads made 4096 x 32768 about 1% slower).
  if constexpr (ROWS == 1) {
    if (!live) return;
  }
  const bool row_live = ROWS == 1 || live;
  const int64_t base = row * nchunk;

  // The row (and residual) chunks first (HBM), then weight and bias (L2 hits).
  u32x4 xv[MAXC], rv[kHasR ? MAXC : 1];
#pragma unroll
  for (int j = 0; j < MAXC; ++j) {
    const int k = j * TPR + t;
    const bool in = row_live && (FULL || k < nchunk);
    xv[j] = in ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.x) + base + k)
               : u32x4{0u, 0u, 0u, 0u};
    if constexpr (kHasR)
      rv[j] = in ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.r) + base + k)
                 : u32x4{0u, 0u, 0u, 0u};
  }
  u32x4 wreg[kHasW ? MAXC : 1], breg[kHasB ? MAXC : 1];
  load_affine<MODE, WPR, MAXC, FULL>(a, t, wreg, breg);

  // Pass 1: sum of squares (LayerNorm: sum). The residual add forms
  // h = round(x + r), stores it and continues with h.
  float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
  for (int j = 0; j < MAXC; ++j) {
    const int k = j * TPR + t;
    if constexpr (kHasR) {
      u32x4 hv;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        hv[e] = DT::pack(DT::lo(xv[j][e]) + DT::lo(rv[j][e]), DT::hi(xv[j][e]) + DT::hi(rv[j][e]));
      xv[j] = hv;
      if (row_live && (FULL || k < nchunk)) store_nt_16(reinterpret_cast<u32x4*>(a.h) + base + k, hv);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p = DT::lo(xv[j][e]);
      const float q = DT::hi(xv[j][e]);
      if constexpr (MODE == Norm::kLayer) {
        acc0 += p;
        acc1 += q;
      } else {
        acc0 = __builtin_fmaf(p, p, acc0);
        acc1 = __builtin_fmaf(q, q, acc1);
      }
    }
  }
  float s1[1] = {acc0 + acc1};
  rows_sum<WPR, 1>(s1, nullptr, &part[slot][0][0], nchunk, t, wave, 0);

  float mu = 0.f, scale;
  if constexpr (MODE == Norm::kLayer) {
    // Pass 1b: centred second moment.
    mu = s1[0] * a.inv_n;
    float c0 = 0.f, c1 = 0.f;
#pragma unroll
    for (int j = 0; j < MAXC; ++j) {
      const int k = j * TPR + t;
      if (FULL || k < nchunk) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = DT::lo(xv[j][e]) - mu;
          const float q = DT::hi(xv[j][e]) - mu;
          c0 = __builtin_fmaf(p, p, c0);
          c1 = __builtin_fmaf(q, q, c1);
        }
      }
    }
    float s2[1] = {c0 + c1};
    rows_sum<WPR, 1>(s2, nullptr, &part[slot][0][0], nchunk, t, wave, 1);
    scale = __builtin_amdgcn_rsqf(s2[0] * a.inv_n + a.eps);
  } else if constexpr (MODE == Norm::kL2) {
    const float nrm = __builtin_sqrtf(s1[0]);
    scale = 1.0f / ((nrm < a.eps) ? a.eps : nrm);  // NaN norms stay NaN
  } else {
    scale = __builtin_amdgcn_rsqf(__builtin_fmaf(s1[0], a.inv_n, a.eps));
  }

  // Pass 2: normalize, weight, round, streaming stores.
  if (!row_live) return;
  u32x4* yrow = reinterpret_cast<u32x4*>(a.y) + base;
#pragma unroll
  for (int j = 0; j < MAXC; ++j) {
    const int k = j * TPR + t;
    if (FULL || k < nchunk) {
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float p = DT::lo(xv[j][e]), q = DT::hi(xv[j][e]);
        if constexpr (MODE == Norm::kLayer) {
          p = __builtin_fmaf((p - mu) * scale, DT::lo(wreg[j][e]), DT::lo(breg[j][e]));
          q = __builtin_fmaf((q - mu) * scale, DT::hi(wreg[j][e]), DT::hi(breg[j][e]));
        } else if constexpr (MODE == Norm::kL2) {
          p *= scale;
          q *= scale;
        } else {
          p = (p * scale) * DT::lo(wreg[j][e]);
          q = (q * scale) * DT::hi(wreg[j][e]);
        }
        o[e] = DT::pack(p, q);
      }
      store_nt_16(yrow + k, o);
    }
  }
}

// Persistent kernel ("[Inductor] Codegen Gluon", section 3.3: copies of the
// next tile in flight while the current one is computed): a grid of at most
// a few workgroups per CU, each looping over row sets g, g + G, g + 2G, ...
// with two LDS buffers. As soon as a row set has landed, the next one's DMA
// is issued into the other buffer, so it overlaps this row set's passes and
// stores; the weight (and bias) registers are loaded once per workgroup.
// Cross-wave partials use a separate [2 parities][2][RPL][WPR] LDS array
// instead of parking: a wave's next DMA refills its own first chunk while
// slower waves may still be reading partials of the previous row set. The
// barrier inside each reduction orders reuse of a parity two row sets later.
// Not for the residual add (its residual registers would need double
// buffering too).
template <Norm MODE, typename DT, int WPR, int RPL, int MAXC, bool FULL>
__global__ void __launch_bounds__(64 * WPR) rownorm_persistent_kernel(RowNormArgs a) {
  static_assert(MODE != Norm::kAddRms, "no persistent residual add");
  constexpr int kPart = 2 * RPL * WPR;  // floats per parity
  extern __shared__ u32x4 lds_rows[];  // 2 * RPL * nchunk chunks, then 2 * kPart floats

  const int nchunk = a.nchunk;
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t sets = (a.M + RPL - 1) / RPL;
  float* part_base = reinterpret_cast<float*>(lds_rows + (size_t)2 * RPL * nchunk);

  u32x4 wreg[Regs<MODE>::kHasW ? MAXC : 1], breg[Regs<MODE>::kHasB ? MAXC : 1];
  load_affine<MODE, WPR, MAXC, FULL>(a, t, wreg, breg);

  int64_t set = blockIdx.x;
  if (set < sets) stage_rows<WPR, RPL, MAXC, FULL>(a, lds_rows, set * RPL, t, wave);
  for (int it = 0; set < sets; set += gridDim.x, ++it) {
    u32x4* cur = lds_rows + (size_t)(it & 1) * RPL * nchunk;
    u32x4* nxt = lds_rows + (size_t)((it + 1) & 1) * RPL * nchunk;
    wait_vmem();  // this row set has landed (and the previous one's stores have completed)
    if (set + gridDim.x < sets) stage_rows<WPR, RPL, MAXC, FULL>(a, nxt, (set + gridDim.x) * RPL, t, wave);
    finish_rows<MODE, DT, WPR, RPL, MAXC, FULL>(a, cur, part_base + (it & 1) * kPart, set * RPL, t, wave,
                                                wreg, breg);
  }
}

typedef void (*RowNormKernel)(RowNormArgs);

// LDS of one CU on gfx950; a workgroup may use all of it.
constexpr size_t kLdsPerCU = 160 * 1024;

struct RowNormCfg {
  int max_nchunk;    // widest row (in 16-byte chunks) this entry serves
  int full_nchunk;   // the kernel's capacity, 64 * wpr * maxc chunks (>= max_nchunk)
  bool exact;        // serves only rows of exactly max_nchunk chunks
  int64_t max_rows;  // serves only launches of at most max_rows rows (0: any)
  int wpr, rows, rpl, maxc;
  int wgs_per_cu;    // occupancy cap (0 = as many as LDS, waves and VGPRs allow)
  int xcd_group;     // row blocks per XCD run (0 = dispatch order)
  RowNormKernel ragged[2];   // any width up to max_nchunk; [bf16, fp16]
  RowNormKernel full[2];     // width exactly full_nchunk; [bf16, fp16]
  RowNormKernel full_cw[2];  // the same with per-chunk waits in pass 1 (_W entries), else null
  bool regs;                 // register-resident rows (rownorm_regs_kernel, _R entries)
};

// A grid of at least this many workgroups (four per CU) takes the per-chunk
// wait kernel of a _W entry: on MI355X it was 1-6% faster there and up to 5%
// slower on smaller grids (12288 x 1536: 768 workgroups).
constexpr int64_t kChunkWaitMinBlocks = 1024;

template <Norm MODE, typename DT, int WPR, int ROWS, int RPL, int MAXC, bool CW>
constexpr RowNormKernel chunk_wait_kernel() {
  if constexpr (CW) return &rownorm_kernel<MODE, DT, WPR, ROWS, RPL, MAXC, true, true>;
  else return nullptr;
}

#define MBN_CFG_(MODE, MAXCH, EXACT, MAXROWS, WPR, ROWS, RPL, MAXC, CAP, GROUP, CW)   \
  RowNormCfg {                                                                        \
    MAXCH, 64 * (WPR) * (MAXC), EXACT, MAXROWS, WPR, ROWS, RPL, MAXC, CAP, GROUP,     \
        {&rownorm_kernel<MODE, Bf16, WPR, ROWS, RPL, MAXC, false>,                    \
         &rownorm_kernel<MODE, F16, WPR, ROWS, RPL, MAXC, false>},                    \
        {&rownorm_kernel<MODE, Bf16, WPR, ROWS, RPL, MAXC, true>,                     \
         &rownorm_kernel<MODE, F16, WPR, ROWS, RPL, MAXC, true>},                     \
        {chunk_wait_kernel<MODE, Bf16, WPR, ROWS, RPL, MAXC, CW>(),                   \
         chunk_wait_kernel<MODE, F16, WPR, ROWS, RPL, MAXC, CW>()},                   \
        false                                                                         \
  }
// serves every width up to 64 * WPR * MAXC chunks (down to the previous entry)
#define MBN_CFG(MODE, WPR, ROWS, RPL, MAXC, CAP, GROUP) \
  MBN_CFG_(MODE, 64 * (WPR) * (MAXC), false, 0, WPR, ROWS, RPL, MAXC, CAP, GROUP, false)
// serves only the width 64 * WPR * MAXC chunks; a later entry covers the band
#define MBN_CFG_EXACT(MODE, WPR, ROWS, RPL, MAXC, CAP, GROUP) \
  MBN_CFG_(MODE, 64 * (WPR) * (MAXC), true, 0, WPR, ROWS, RPL, MAXC, CAP, GROUP, false)
// serves the widths of the band that ends at 64 * WPR * MAXC chunks, for
// launches of at most MAXROWS rows (row windows precede the band's entry for
// any row count, in increasing MAXROWS)
#define MBN_CFG_ROWS(MODE, MAXROWS, WPR, ROWS, RPL, MAXC, CAP, GROUP) \
  MBN_CFG_(MODE, 64 * (WPR) * (MAXC), false, MAXROWS, WPR, ROWS, RPL, MAXC, CAP, GROUP, false)
// a row window that serves only the width 64 * WPR * MAXC chunks (the band's
// top width); placed after other windows it holds their row counts for that
// width only, so that a later exact window starts above them
#define MBN_CFG_ROWS_EXACT(MODE, MAXROWS, WPR, ROWS, RPL, MAXC, CAP, GROUP) \
  MBN_CFG_(MODE, 64 * (WPR) * (MAXC), true, MAXROWS, WPR, ROWS, RPL, MAXC, CAP, GROUP, false)
// the same with per-chunk waits
#define MBN_CFG_ROWS_EXACT_W(MODE, MAXROWS, WPR, ROWS, RPL, MAXC, CAP, GROUP) \
  MBN_CFG_(MODE, 64 * (WPR) * (MAXC), true, MAXROWS, WPR, ROWS, RPL, MAXC, CAP, GROUP, true)
// sub-band: serves the widths from the band's lower edge (or the previous
// sub-band) up to MAXN elements, MAXN / 8 <= 64 * WPR * MAXC, at the row
// counts the band's row windows leave; sub-bands follow the band's windows
// and precede its entry, in increasing MAXN
#define MBN_CFG_UPTO(MODE, MAXN, WPR, ROWS, RPL, MAXC, CAP, GROUP) \
  MBN_CFG_(MODE, (MAXN) / 8, false, 0, WPR, ROWS, RPL, MAXC, CAP, GROUP, false)
// The _W forms: the same entries with a second full-width kernel that takes
// each staged chunk as it lands (per-chunk waits in pass 1), used for grids of
// at least kChunkWaitMinBlocks workgroups
#define MBN_CFG_W(MODE, WPR, ROWS, RPL, MAXC, CAP, GROUP) \
  MBN_CFG_(MODE, 64 * (WPR) * (MAXC), false, 0, WPR, ROWS, RPL, MAXC, CAP, GROUP, true)
#define MBN_CFG_EXACT_W(MODE, WPR, ROWS, RPL, MAXC, CAP, GROUP) \
  MBN_CFG_(MODE, 64 * (WPR) * (MAXC), true, 0, WPR, ROWS, RPL, MAXC, CAP, GROUP, true)
#define MBN_CFG_UPTO_W(MODE, MAXN, WPR, ROWS, RPL, MAXC, CAP, GROUP) \
  MBN_CFG_(MODE, (MAXN) / 8, false, 0, WPR, ROWS, RPL, MAXC, CAP, GROUP, true)

// The _LW form: a band's entry whose kernels load the weight (and bias) after
// the reduction (rownorm_lw_kernel), for grids of any size.
#define MBN_CFG_LW(MODE, WPR, ROWS, RPL, MAXC, CAP, GROUP)                              \
  RowNormCfg {                                                                        \
    64 * (WPR) * (MAXC), 64 * (WPR) * (MAXC), false, 0, WPR, ROWS, RPL, MAXC, CAP, GROUP, \
        {&rownorm_lw_kernel<MODE, Bf16, WPR, ROWS, RPL, MAXC, false>,                 \
         &rownorm_lw_kernel<MODE, F16, WPR, ROWS, RPL, MAXC, false>},                 \
        {&rownorm_lw_kernel<MODE, Bf16, WPR, ROWS, RPL, MAXC, true>,                  \
         &rownorm_lw_kernel<MODE, F16, WPR, ROWS, RPL, MAXC, true>},                  \
        {nullptr, nullptr}, false                                                     \
  }

// The _R form: an exact-width entry with register-resident rows
// (rownorm_regs_kernel: one row per lane set, RPL = 1, no LDS staging; CAP
// still caps the resident workgroups per CU through the dynamic LDS request).
// Only exact widths: at widths below a kernel's capacity it measured 10-12%
// slower than the staged kernel; and only past a row window that keeps the
// staged kernel for launches of up to 1536-2048 rows, where it was 3-9%
// slower.
#define MBN_CFG_EXACT_R(MODE, WPR, ROWS, MAXC, CAP, GROUP)                             \
  RowNormCfg {                                                                       \
    64 * (WPR) * (MAXC), 64 * (WPR) * (MAXC), true, 0, WPR, ROWS, 1, MAXC, CAP, GROUP, \
        {nullptr, nullptr},                                                          \
        {&rownorm_regs_kernel<MODE, Bf16, WPR, ROWS, MAXC, true>,                    \
         &rownorm_regs_kernel<MODE, F16, WPR, ROWS, MAXC, true>},                    \
        {nullptr, nullptr}, true                                                     \
  }

// The _ROWS_R form: a row window with register-resident rows at one exact
// width (rownorm_regs_kernel, RPL = 1) for small launches. On MI355X, at
// N = 2048 ... 16384 and a few hundred to two thousand rows, the kernel-trace
// medians of these geometries were 2-38% below the staged kernels' windows
// (RMSNorm 3-12%, LayerNorm, L2Norm and the residual add per width and row
// count, each window kept only where two runs agreed): a small launch's time
// is mostly the latency of one row's trip, and the rows go HBM -> VGPRs
// without the LDS write and read. Windows are listed before the
// band's other windows (they serve only its top width), in increasing MAXROWS.
#define MBN_CFG_ROWS_EXACT_R(MODE, MAXROWS, WPR, ROWS, MAXC, CAP, GROUP)                       \
  RowNormCfg {                                                                                \
    64 * (WPR) * (MAXC), 64 * (WPR) * (MAXC), true, MAXROWS, WPR, ROWS, 1, MAXC, CAP, GROUP,    \
        {nullptr, nullptr},                                                                   \
        {&rownorm_regs_kernel<MODE, Bf16, WPR, ROWS, MAXC, true>,                             \
         &rownorm_regs_kernel<MODE, F16, WPR, ROWS, MAXC, true>},                             \
        {nullptr, nullptr}, true                                                              \
  }

// Per-width launch tables, narrowest first: the first entry that serves the
// row width is used. Every entry with WPR > 1 serves only widths of at least
// 64 * WPR chunks, which the parked partial sums need (exact entries, or the
// previous band ending at or above 64 * WPR).
//
// Entries for N = 1024 ... 65536 were chosen by timing every shape / cap /
// group combination of the kernel template on MI355X at M * N = 2^26, 2^27
// and 2^28 (buffers rotated over >= 1 GiB, so nothing is served from the
// 256 MiB Infinity Cache), taking the best geometric mean over the three;
// RMSNorm at N = 16384 keeps the entry that is fastest at M = 16384. The
// N <= 512 band is untuned. Row windows (MBN_CFG_ROWS) come from the same
// timing at N = 1024 ... 32768 and M = 256 ... 32768 with M * N < 2^26: the
// sampled row counts of a band were split into windows, each given the
// configuration with the least total log-time over its rows that is nowhere
// more than 1% slower than the band's general entry, at a cost of 5% per
// window (so a window must pay for itself); launches of more rows than the
// last window use the general entry. An A/B of the library against the
// tables without windows (GPU kernel durations, both orders, at widths and
// row counts between the sampled ones too) then shortened the residual-add
// and L2Norm windows that were slower there. Sub-bands (MBN_CFG_UPTO) and
// exact widths between powers of two: the band entries are tuned at the
// band's top width, and between powers of two another geometry often did
// better. From timing every tight geometry at N = 5120 ... 18432 (M * N =
// 2^26, 2^27 and 2^28, rotated buffers): each such entry was nowhere more than
// 1% slower than the band entry at the widths timed inside it and 2-10%
// faster at most of them (RMSNorm sub-bands also timed at 4352 ... 6144,
// 8448 ... 15360 and 16896 ... 19456; the RMSNorm one up to 6144 is within
// 1% at 6144 itself).
#define MBN_FIRST_BAND(MODE) MBN_CFG(MODE, 1, 4, 1, 1, 0, 0) /* N <= 512 */

const RowNormCfg kRmsTable[] = {
    MBN_FIRST_BAND(Norm::kRms),
    MBN_CFG_ROWS(Norm::kRms, 2048, 1, 4, 1, 2, 0, 0),  // N <= 1024, M <= 2048
    MBN_CFG_ROWS(Norm::kRms, 8192, 1, 4, 2, 2, 4, 0),  // N <= 1024, M <= 8192
    MBN_CFG(Norm::kRms, 1, 4, 1, 2, 0, 16),  // N <= 1024:  4 x 64 threads
    MBN_CFG_ROWS_EXACT_R(Norm::kRms, 1024, 1, 1, 4, 0, 0),  // N == 2048, M <= 1024: 64 lanes, rows in VGPRs
    MBN_CFG_ROWS_EXACT_R(Norm::kRms, 1536, 2, 1, 2, 0, 0),  // N == 2048, M <= 1536: 128 lanes, rows in VGPRs
    MBN_CFG_ROWS_EXACT_R(Norm::kRms, 2048, 1, 4, 4, 0, 0),  // N == 2048, M <= 2048: 4 x 64 lanes, rows in VGPRs
    MBN_CFG_ROWS(Norm::kRms, 256, 2, 2, 1, 2, 1, 0),  // N <= 2048, M <= 256
    MBN_CFG_ROWS(Norm::kRms, 2048, 1, 4, 1, 4, 4, 0),  // N <= 2048, M <= 2048
    MBN_CFG_ROWS(Norm::kRms, 4096, 1, 4, 2, 4, 2, 0),  // N <= 2048, M <= 4096
    MBN_CFG(Norm::kRms, 2, 2, 2, 2, 4, 8),   // N <= 2048:  2 x 128 threads x 2 rows, 4 WGs/CU
    MBN_CFG_ROWS_EXACT_R(Norm::kRms, 512, 4, 1, 2, 0, 0),  // N == 4096, M <= 512: 256 lanes, rows in VGPRs
    MBN_CFG_ROWS_EXACT_R(Norm::kRms, 2048, 1, 1, 8, 0, 0),  // N == 4096, M <= 2048: 64 lanes, rows in VGPRs
    MBN_CFG_ROWS_EXACT_R(Norm::kRms, 4096, 1, 2, 8, 0, 0),  // N == 4096, M <= 4096: 2 x 64 lanes, rows in VGPRs
    MBN_CFG_ROWS(Norm::kRms, 512, 4, 1, 1, 2, 0, 0),  // N <= 4096, M <= 512
    MBN_CFG_ROWS(Norm::kRms, 1024, 2, 2, 1, 4, 3, 0),  // N <= 4096, M <= 1024
    MBN_CFG_ROWS(Norm::kRms, 4096, 2, 1, 2, 4, 0, 0),  // N <= 4096, M <= 4096
    MBN_CFG_W(Norm::kRms, 4, 1, 2, 2, 4, 8),   // N <= 4096:  256 threads x 2 rows, 4 WGs/CU
    MBN_CFG_ROWS_EXACT_R(Norm::kRms, 256, 4, 1, 4, 0, 0),  // N == 8192, M <= 256: 256 lanes, rows in VGPRs
    MBN_CFG_ROWS_EXACT_R(Norm::kRms, 512, 4, 2, 4, 0, 0),  // N == 8192, M <= 512: 2 x 256 lanes, rows in VGPRs
    MBN_CFG_ROWS_EXACT_R(Norm::kRms, 768, 2, 1, 8, 0, 0),  // N == 8192, M <= 768: 128 lanes, rows in VGPRs
    MBN_CFG_ROWS_EXACT_R(Norm::kRms, 1024, 4, 2, 4, 0, 0),  // N == 8192, M <= 1024: 2 x 256 lanes, rows in VGPRs
    MBN_CFG_ROWS(Norm::kRms, 512, 4, 1, 1, 4, 0, 0),  // N <= 8192, M <= 512
    MBN_CFG_ROWS(Norm::kRms, 1024, 2, 1, 1, 8, 0, 0),  // N <= 8192, M <= 1024
    MBN_CFG_ROWS(Norm::kRms, 2048, 2, 1, 2, 8, 0, 0),  // N <= 8192, M <= 2048
    MBN_CFG_EXACT_W(Norm::kRms, 4, 1, 2, 3, 2, 0),  // N == 6144: 256 threads x 2 rows
    MBN_CFG_UPTO(Norm::kRms, 6144, 6, 1, 2, 2, 4, 0),  // 4096 < N <= 6144: 384 threads x 2 rows
    MBN_CFG_EXACT_W(Norm::kRms, 7, 1, 2, 2, 3, 0),  // N == 7168: 448 threads x 2 rows
    MBN_CFG_LW(Norm::kRms, 8, 1, 1, 2, 0, 0),  // N <= 8192:  512 threads, weight after the reduction
    MBN_CFG_ROWS_EXACT_R(Norm::kRms, 256, 8, 1, 4, 0, 0),  // N == 16384, M <= 256: 512 lanes, rows in VGPRs
    MBN_CFG_ROWS_EXACT_R(Norm::kRms, 512, 8, 2, 4, 0, 0),  // N == 16384, M <= 512: 2 x 512 lanes, rows in VGPRs
    MBN_CFG_ROWS_EXACT_R(Norm::kRms, 768, 4, 1, 8, 0, 0),  // N == 16384, M <= 768: 256 lanes, rows in VGPRs
    MBN_CFG_ROWS(Norm::kRms, 256, 16, 1, 1, 2, 0, 0),  // N <= 16384, M <= 256
    MBN_CFG_ROWS(Norm::kRms, 1536, 4, 1, 2, 8, 0, 0),  // N <= 16384, M <= 1536
    MBN_CFG_ROWS_EXACT_W(Norm::kRms, 6144, 4, 1, 1, 8, 2, 8),  // N == 16384, M <= 6144
    MBN_CFG_UPTO_W(Norm::kRms, 12288, 12, 1, 2, 2, 0, 0),  // 8192 < N <= 12288: 768 threads x 2 rows
    MBN_CFG_UPTO(Norm::kRms, 15360, 16, 1, 2, 2, 0, 0),  // 12288 < N <= 15360: 1024 threads x 2 rows
    MBN_CFG_W(Norm::kRms, 2, 2, 1, 16, 2, 4),  // N <= 16384: 2 x 128 threads, 2 WGs/CU
    MBN_CFG_ROWS_EXACT_W(Norm::kRms, 2048, 16, 1, 1, 4, 0, 0),  // N == 32768, M <= 2048: rows in LDS
    MBN_CFG_EXACT_R(Norm::kRms, 16, 1, 4, 4, 4),  // N == 32768: 1024 threads, rows in VGPRs
    MBN_CFG_UPTO(Norm::kRms, 19456, 8, 1, 1, 5, 3, 0),  // 16384 < N <= 19456: 512 threads
    MBN_CFG(Norm::kRms, 16, 1, 1, 4, 0, 0),  // N < 32768: 1024 threads (the top width: the two entries above)
    MBN_CFG_ROWS_EXACT_W(Norm::kRms, 1536, 16, 1, 1, 8, 0, 0),  // N == 65536, M <= 1536: rows in LDS
    MBN_CFG_EXACT_R(Norm::kRms, 8, 1, 16, 4, 4),  // N == 65536: 512 threads, rows in VGPRs
    MBN_CFG(Norm::kRms, 16, 1, 1, 8, 0, 0),  // N < 65536: 1024 threads (the top width: the two entries above)
};
const RowNormCfg kAddRmsTable[] = {
    MBN_FIRST_BAND(Norm::kAddRms),
    MBN_CFG_ROWS(Norm::kAddRms, 4096, 1, 4, 1, 2, 0, 0),  // N <= 1024, M <= 4096
    MBN_CFG_ROWS(Norm::kAddRms, 32768, 1, 4, 2, 2, 0, 0),  // N <= 1024, M <= 32768
    MBN_CFG(Norm::kAddRms, 1, 4, 1, 2, 4, 16),  // N <= 1024
    MBN_CFG_ROWS_EXACT_R(Norm::kAddRms, 768, 2, 1, 2, 0, 0),  // N == 2048, M <= 768: 128 lanes, rows in VGPRs
    MBN_CFG_ROWS_EXACT_R(Norm::kAddRms, 1024, 4, 1, 1, 0, 0),  // N == 2048, M <= 1024: 256 lanes, rows in VGPRs
    MBN_CFG_ROWS_EXACT_R(Norm::kAddRms, 1536, 2, 1, 2, 0, 0),  // N == 2048, M <= 1536: 128 lanes, rows in VGPRs
    MBN_CFG_ROWS_EXACT_R(Norm::kAddRms, 2048, 1, 4, 4, 0, 0),  // N == 2048, M <= 2048: 4 x 64 lanes, rows in VGPRs
    MBN_CFG_ROWS(Norm::kAddRms, 1024, 2, 2, 1, 2, 0, 0),  // N <= 2048, M <= 1024
    MBN_CFG_ROWS(Norm::kAddRms, 8192, 2, 2, 2, 2, 4, 0),  // N <= 2048, M <= 8192
    MBN_CFG(Norm::kAddRms, 1, 4, 1, 4, 2, 8),   // N <= 2048
    MBN_CFG_ROWS_EXACT_R(Norm::kAddRms, 768, 8, 1, 1, 0, 0),  // N == 4096, M <= 768: 512 lanes, rows in VGPRs
    MBN_CFG_ROWS_EXACT_R(Norm::kAddRms, 1024, 4, 2, 2, 0, 0),  // N == 4096, M <= 1024: 2 x 256 lanes, rows in VGPRs
    MBN_CFG_ROWS_EXACT_R(Norm::kAddRms, 1536, 1, 2, 8, 0, 0),  // N == 4096, M <= 1536: 2 x 64 lanes, rows in VGPRs
    MBN_CFG_ROWS(Norm::kAddRms, 256, 4, 1, 1, 2, 4, 0),  // N <= 4096, M <= 256
    MBN_CFG_ROWS(Norm::kAddRms, 512, 4, 2, 1, 2, 0, 16),  // N <= 4096, M <= 512
    MBN_CFG_ROWS(Norm::kAddRms, 1024, 4, 1, 1, 2, 4, 16),  // N <= 4096, M <= 1024 (the band's general entry)
    MBN_CFG_ROWS(Norm::kAddRms, 4096, 1, 4, 1, 8, 0, 0),  // N <= 4096, M <= 4096
    MBN_CFG(Norm::kAddRms, 4, 1, 1, 2, 4, 16),  // N <= 4096:  256 threads, 4 WGs/CU
    MBN_CFG_ROWS_EXACT_R(Norm::kAddRms, 256, 16, 1, 1, 0, 0),  // N == 8192, M <= 256: 1024 lanes, rows in VGPRs
    MBN_CFG_ROWS_EXACT_R(Norm::kAddRms, 512, 4, 2, 4, 0, 0),  // N == 8192, M <= 512: 2 x 256 lanes, rows in VGPRs
    MBN_CFG_ROWS(Norm::kAddRms, 256, 8, 1, 1, 2, 1, 64),  // N <= 8192, M <= 256
    MBN_CFG_ROWS(Norm::kAddRms, 512, 8, 1, 2, 2, 0, 0),  // N <= 8192, M <= 512
    MBN_CFG_ROWS_EXACT(Norm::kAddRms, 1024, 2, 1, 1, 8, 0, 0),  // N == 8192, M <= 1024: the next window's kernel
    MBN_CFG_ROWS_EXACT_R(Norm::kAddRms, 1536, 2, 2, 8, 0, 0),  // N == 8192, M <= 1536: 2 x 128 lanes, rows in VGPRs
    MBN_CFG_ROWS(Norm::kAddRms, 2048, 2, 1, 1, 8, 0, 0),  // N <= 8192, M <= 2048
    MBN_CFG_EXACT(Norm::kAddRms, 2, 2, 1, 5, 2, 4),  // N == 5120: 2 x 128 threads
    MBN_CFG(Norm::kAddRms, 8, 1, 1, 2, 2, 8),   // N <= 8192:  512 threads, 2 WGs/CU
    MBN_CFG_ROWS_EXACT_R(Norm::kAddRms, 256, 4, 1, 8, 0, 0),  // N == 16384, M <= 256: 256 lanes, rows in VGPRs
    MBN_CFG_ROWS(Norm::kAddRms, 256, 8, 1, 1, 4, 4, 0),  // N <= 16384, M <= 256
    MBN_CFG_ROWS(Norm::kAddRms, 512, 8, 1, 2, 4, 0, 0),  // N <= 16384, M <= 512
    MBN_CFG_ROWS(Norm::kAddRms, 1024, 16, 1, 4, 2, 0, 0),  // N <= 16384, M <= 1024
    MBN_CFG_ROWS_EXACT_R(Norm::kAddRms, 2048, 16, 1, 2, 0, 0),  // N == 16384, M <= 2048: 1024 lanes, rows in VGPRs
    MBN_CFG(Norm::kAddRms, 4, 1, 1, 8, 3, 4),   // N <= 16384: 256 threads, 3 WGs/CU
    MBN_CFG_ROWS(Norm::kAddRms, 512, 4, 1, 1, 16, 2, 0),  // N <= 32768, M <= 512
    MBN_CFG(Norm::kAddRms, 16, 1, 1, 4, 2, 2),  // N <= 32768: 1024 threads
    MBN_CFG(Norm::kAddRms, 16, 1, 1, 8, 0, 0),  // N <= 65536
};
const RowNormCfg kLayerTable[] = {
    MBN_FIRST_BAND(Norm::kLayer),
    MBN_CFG_ROWS(Norm::kLayer, 2048, 1, 4, 1, 2, 0, 0),  // N <= 1024, M <= 2048
    MBN_CFG(Norm::kLayer, 1, 4, 2, 2, 4, 0),   // N <= 1024
    MBN_CFG_ROWS_EXACT_R(Norm::kLayer, 1536, 1, 1, 4, 0, 0),  // N == 2048, M <= 1536: 64 lanes, rows in VGPRs
    MBN_CFG_ROWS_EXACT_R(Norm::kLayer, 2048, 1, 2, 4, 0, 0),  // N == 2048, M <= 2048: 2 x 64 lanes, rows in VGPRs
    MBN_CFG_ROWS(Norm::kLayer, 2048, 2, 2, 1, 2, 0, 0),  // N <= 2048, M <= 2048
    MBN_CFG_ROWS(Norm::kLayer, 4096, 1, 4, 2, 4, 0, 0),  // N <= 2048, M <= 4096
    MBN_CFG(Norm::kLayer, 2, 2, 2, 2, 4, 8),   // N <= 2048
    MBN_CFG_ROWS_EXACT_R(Norm::kLayer, 256, 4, 1, 2, 0, 0),  // N == 4096, M <= 256: 256 lanes, rows in VGPRs
    MBN_CFG_ROWS_EXACT_R(Norm::kLayer, 384, 4, 2, 2, 0, 0),  // N == 4096, M <= 384: 2 x 256 lanes, rows in VGPRs
    MBN_CFG_ROWS_EXACT_R(Norm::kLayer, 1024, 1, 1, 8, 0, 0),  // N == 4096, M <= 1024: 64 lanes, rows in VGPRs
    MBN_CFG_ROWS_EXACT_R(Norm::kLayer, 2048, 2, 2, 4, 0, 0),  // N == 4096, M <= 2048: 2 x 128 lanes, rows in VGPRs
    MBN_CFG_ROWS_EXACT_R(Norm::kLayer, 3072, 1, 2, 8, 0, 0),  // N == 4096, M <= 3072: 2 x 64 lanes, rows in VGPRs
    MBN_CFG_ROWS(Norm::kLayer, 512, 4, 1, 1, 2, 4, 2),  // N <= 4096, M <= 512
    MBN_CFG_ROWS(Norm::kLayer, 1024, 4, 2, 1, 2, 2, 0),  // N <= 4096, M <= 1024
    MBN_CFG_ROWS(Norm::kLayer, 2048, 1, 4, 1, 8, 2, 0),  // N <= 4096, M <= 2048
    MBN_CFG_W(Norm::kLayer, 4, 1, 2, 2, 4, 8),   // N <= 4096:  256 threads x 2 rows
    MBN_CFG_ROWS_EXACT_R(Norm::kLayer, 512, 4, 1, 4, 0, 0),  // N == 8192, M <= 512: 256 lanes, rows in VGPRs
    MBN_CFG_ROWS_EXACT_R(Norm::kLayer, 1536, 2, 1, 8, 0, 0),  // N == 8192, M <= 1536: 128 lanes, rows in VGPRs
    MBN_CFG_ROWS(Norm::kLayer, 512, 8, 1, 1, 2, 3, 0),  // N <= 8192, M <= 512
    MBN_CFG_ROWS(Norm::kLayer, 1024, 4, 1, 2, 4, 2, 0),  // N <= 8192, M <= 1024
    MBN_CFG_ROWS(Norm::kLayer, 2048, 8, 1, 4, 2, 2, 0),  // N <= 8192, M <= 2048
    MBN_CFG_EXACT_W(Norm::kLayer, 2, 2, 2, 5, 3, 0),  // N == 5120: 2 x 128 threads x 2 rows
    MBN_CFG_EXACT_W(Norm::kLayer, 4, 1, 2, 3, 3, 0),  // N == 6144: 256 threads x 2 rows
    MBN_CFG_EXACT_W(Norm::kLayer, 2, 2, 2, 7, 2, 0),  // N == 7168: 2 x 128 threads x 2 rows
    MBN_CFG_W(Norm::kLayer, 8, 1, 2, 2, 4, 16),  // N <= 8192:  512 threads x 2 rows
    MBN_CFG_ROWS_EXACT_R(Norm::kLayer, 256, 8, 1, 4, 0, 0),  // N == 16384, M <= 256: 512 lanes, rows in VGPRs
    MBN_CFG_ROWS_EXACT_R(Norm::kLayer, 768, 4, 1, 8, 0, 0),  // N == 16384, M <= 768: 256 lanes, rows in VGPRs
    MBN_CFG_ROWS(Norm::kLayer, 512, 16, 1, 1, 2, 2, 0),  // N <= 16384, M <= 512
    MBN_CFG_ROWS(Norm::kLayer, 1024, 4, 1, 2, 8, 2, 0),  // N <= 16384, M <= 1024
    MBN_CFG_EXACT_W(Norm::kLayer, 4, 1, 2, 5, 3, 8),  // N == 10240: 256 threads x 2 rows
    MBN_CFG_EXACT_W(Norm::kLayer, 4, 1, 2, 6, 2, 0),  // N == 12288
    MBN_CFG_EXACT_W(Norm::kLayer, 4, 1, 2, 7, 2, 0),  // N == 14336
    MBN_CFG_EXACT_W(Norm::kLayer, 4, 1, 2, 8, 2, 4),  // N == 16384: 256 threads x 2 rows
    MBN_CFG_W(Norm::kLayer, 2, 2, 1, 16, 0, 0),  // N <= 16384: 2 x 128 threads
    MBN_CFG_ROWS(Norm::kLayer, 256, 8, 1, 1, 8, 1, 0),  // N <= 32768, M <= 256
    MBN_CFG(Norm::kLayer, 4, 1, 1, 16, 0, 4),  // N <= 32768: 256 threads
    MBN_CFG_W(Norm::kLayer, 8, 1, 1, 16, 1, 0),  // N <= 65536: 512 threads
};
const RowNormCfg kL2Table[] = {
    MBN_FIRST_BAND(Norm::kL2),
    MBN_CFG_ROWS(Norm::kL2, 2048, 1, 4, 1, 2, 0, 0),  // N <= 1024, M <= 2048
    MBN_CFG(Norm::kL2, 1, 4, 2, 2, 4, 0),   // N <= 1024
    MBN_CFG_ROWS_EXACT_R(Norm::kL2, 768, 1, 1, 4, 0, 0),  // N == 2048, M <= 768: 64 lanes, rows in VGPRs
    MBN_CFG_ROWS_EXACT_R(Norm::kL2, 1536, 2, 1, 2, 0, 0),  // N == 2048, M <= 1536: 128 lanes, rows in VGPRs
    MBN_CFG_ROWS(Norm::kL2, 1024, 1, 4, 1, 4, 4, 0),  // N <= 2048, M <= 1024
    MBN_CFG(Norm::kL2, 2, 2, 2, 2, 4, 0),   // N <= 2048
    MBN_CFG_ROWS(Norm::kL2, 768, 4, 1, 1, 2, 0, 0),  // N <= 4096, M <= 768
    MBN_CFG(Norm::kL2, 2, 2, 1, 4, 4, 0),   // N <= 4096:  2 x 128 threads
    MBN_CFG_ROWS(Norm::kL2, 1024, 8, 1, 1, 2, 0, 0),  // N <= 8192, M <= 1024
    MBN_CFG_ROWS_EXACT_R(Norm::kL2, 1536, 2, 2, 8, 0, 0),  // N == 8192, M <= 1536: 2 x 128 lanes, rows in VGPRs
    MBN_CFG_ROWS(Norm::kL2, 2048, 8, 1, 4, 2, 0, 0),  // N <= 8192, M <= 2048
    MBN_CFG(Norm::kL2, 8, 1, 1, 2, 0, 0),   // N <= 8192:  512 threads
    MBN_CFG_ROWS_EXACT(Norm::kL2, 256, 8, 1, 1, 4, 2, 0),  // N == 16384, M <= 256: the M <= 512 window's kernel
    MBN_CFG_ROWS_EXACT_R(Norm::kL2, 384, 8, 2, 4, 0, 0),  // N == 16384, M <= 384: 2 x 512 lanes, rows in VGPRs
    MBN_CFG_ROWS(Norm::kL2, 512, 8, 1, 1, 4, 2, 0),  // N <= 16384, M <= 512
    MBN_CFG_ROWS_EXACT(Norm::kL2, 1024, 2, 2, 1, 16, 2, 0),  // N == 16384, M <= 1024: the M <= 2048 window's kernel
    MBN_CFG_ROWS_EXACT_R(Norm::kL2, 2048, 4, 1, 8, 0, 0),  // N == 16384, M <= 2048: 256 lanes, rows in VGPRs
    MBN_CFG_ROWS(Norm::kL2, 2048, 2, 2, 1, 16, 2, 0),  // N <= 16384, M <= 2048
    MBN_CFG_UPTO(Norm::kL2, 12288, 12, 1, 1, 2, 3, 0),  // 8192 < N <= 12288: 768 threads
    MBN_CFG(Norm::kL2, 4, 1, 1, 8, 3, 4),   // N <= 16384: 256 threads, 3 WGs/CU
    MBN_CFG_ROWS(Norm::kL2, 256, 8, 1, 1, 8, 2, 0),  // N <= 32768, M <= 256
    MBN_CFG_ROWS(Norm::kL2, 1024, 4, 1, 1, 16, 2, 16),  // N <= 32768, M <= 1024
    MBN_CFG(Norm::kL2, 16, 1, 1, 4, 0, 8),  // N <= 32768: 1024 threads
    MBN_CFG(Norm::kL2, 16, 1, 1, 8, 0, 0),  // N <= 65536
};

template <size_t K>
const RowNormCfg* pick(const RowNormCfg (&table)[K], int nchunk, int64_t M) {
  for (const RowNormCfg& c : table)
    if ((c.exact ? nchunk == c.max_nchunk : nchunk <= c.max_nchunk) && (c.max_rows == 0 || M <= c.max_rows))
      return &c;
  return nullptr;
}


// Persistent launches (rownorm_persistent_kernel) for the middle widths, for
// RMSNorm, LayerNorm and L2Norm: an entry serves widths [min_nchunk,
// max_nchunk] (chunks) at row counts [min_rows, max_rows]; the first entry
// that matches is used, else the one-shot table. Entries and windows come from
// an interleaved timing sweep on MI355X against the one-shot tables (row
// windows included): N = 2560 ... 8192, M = 256 ... 8192, grids of 512 ...
// 2048 workgroups, cold and warm caches. The persistent kernel is used at a
// sampled row count where, at every measured width of the band and with both
// caches, it took at most 98% of the one-shot time (typically 80-95%); a
// window ends half way (geometrically) between such a row count and one where
// it lost. The best grid keeps about 40-64 KiB of row copies in flight per CU.
struct PersistentCfg {
  int min_nchunk, max_nchunk;  // widths served, in 16-byte chunks
  int wpr, rpl, maxc;
  int grid;                    // workgroups launched (fewer if there are fewer row sets)
  int64_t min_rows, max_rows;  // row counts served
  RowNormKernel ragged[2];     // [bf16, fp16]
  RowNormKernel full[2];       // width exactly 64 * wpr * maxc chunks
};

#define MBN_PCFG(MODE, LO, HI, WPR, RPL, MAXC, GRID, MINROWS, MAXROWS)                \
  PersistentCfg {                                                                     \
    LO, HI, WPR, RPL, MAXC, GRID, MINROWS, MAXROWS,                                   \
        {&rownorm_persistent_kernel<MODE, Bf16, WPR, RPL, MAXC, false>,               \
         &rownorm_persistent_kernel<MODE, F16, WPR, RPL, MAXC, false>},               \
        {&rownorm_persistent_kernel<MODE, Bf16, WPR, RPL, MAXC, true>,                \
         &rownorm_persistent_kernel<MODE, F16, WPR, RPL, MAXC, true>}                 \
  }

const PersistentCfg kRmsPersistent[] = {
    MBN_PCFG(Norm::kRms, 257, 384, 4, 1, 2, 2048, 725, 1448),   // 2048 < N <= 3072
    MBN_PCFG(Norm::kRms, 257, 384, 4, 1, 2, 2048, 5017, 8192),
    MBN_PCFG(Norm::kRms, 385, 512, 4, 1, 2, 1536, 2509, 8192),  // 3072 < N <= 4096
    MBN_PCFG(Norm::kRms, 513, 768, 4, 1, 4, 1024, 1449, 7094),  // 4096 < N <= 6144
    MBN_PCFG(Norm::kRms, 769, 1024, 4, 1, 4, 1024, 2509, 3547),  // 6144 < N <= 8192
};
const PersistentCfg kLayerPersistent[] = {
    MBN_PCFG(Norm::kLayer, 257, 384, 4, 1, 2, 1536, 1, 8192),
    MBN_PCFG(Norm::kLayer, 385, 512, 4, 1, 2, 1536, 725, 1448),
    MBN_PCFG(Norm::kLayer, 385, 512, 4, 1, 2, 1536, 2509, 5017),
    MBN_PCFG(Norm::kLayer, 513, 768, 4, 1, 4, 1024, 725, 8192),
    MBN_PCFG(Norm::kLayer, 769, 1024, 4, 1, 4, 1024, 2509, 5017),
};
const PersistentCfg kL2Persistent[] = {
    MBN_PCFG(Norm::kL2, 257, 384, 4, 1, 2, 2048, 363, 1448),
    MBN_PCFG(Norm::kL2, 257, 384, 4, 1, 2, 2048, 2509, 7094),
    MBN_PCFG(Norm::kL2, 513, 768, 4, 1, 4, 1024, 725, 1448),
};

template <size_t K>
const PersistentCfg* pick_persistent(const PersistentCfg (&table)[K], int nchunk, int64_t M,
                                     bool any_rows) {
  for (const PersistentCfg& c : table)
    if (nchunk >= c.min_nchunk && nchunk <= c.max_nchunk &&
        (any_rows || (M >= c.min_rows && M <= c.max_rows)))
      return &c;
  return nullptr;
}

// LDS of a persistent launch: two buffers of RPL rows, then the partials
// ([2 parities][2 reductions][RPL][WPR] floats).
size_t persistent_lds_bytes(const PersistentCfg& c, int nchunk) {
  return (size_t)2 * c.rpl * nchunk * 16 + (size_t)4 * c.rpl * c.wpr * sizeof(float);
}
}  // namespace

// Dynamic LDS of a launch: the staged rows, raised to kLdsPerCU / cap when an
// occupancy cap asks for fewer resident workgroups per CU than LDS would allow.
size_t rownorm_lds_bytes(int rows, int64_t N, int wgs_per_cu) {
  size_t lds = (size_t)rows * (size_t)N * 2;
  if (wgs_per_cu > 0) {
    const size_t cap = (kLdsPerCU / (size_t)wgs_per_cu) & ~(size_t)511;
    if (cap > lds) lds = cap;
  }
  return lds;
}

// Dynamic LDS of a register-resident launch: none, or enough to hold the
// resident workgroups per CU to the cap (kLdsPerCU / cap, less room for the
// kernel's static partial sums, at most 512 bytes).
size_t rownorm_regs_lds_bytes(int wgs_per_cu) {
  if (wgs_per_cu <= 0) return 0;
  return ((kLdsPerCU / (size_t)wgs_per_cu) & ~(size_t)511) - 1024;
}

hipError_t launch_rownorm(Norm mode, Storage dtype, RowNormArgs args, hipStream_t stream,
                          RowNormPath path, int grid) {
  const int nchunk = args.nchunk;
  const int64_t N = (int64_t)nchunk * 8;
  const int d = dtype == Storage::kF16 ? 1 : 0;
  args.inv_n = 1.0f / (float)N;
  args.xcd_group = 0;

  const RowNormCfg* cfg = nullptr;
  switch (mode) {
    case Norm::kRms: cfg = pick(kRmsTable, nchunk, args.M); break;
    case Norm::kAddRms: cfg = pick(kAddRmsTable, nchunk, args.M); break;
    case Norm::kLayer: cfg = pick(kLayerTable, nchunk, args.M); break;
    case Norm::kL2: cfg = pick(kL2Table, nchunk, args.M); break;
  }
  // An exact-width register-row window serves its launches ahead of the
  // persistent table: those windows were chosen against whatever served the
  // launch before, the persistent kernel included.
  const bool regs_window = cfg && cfg->regs && cfg->max_rows > 0;

  if (path == RowNormPath::kPersistent || (path == RowNormPath::kAuto && !regs_window)) {
    const bool forced = path == RowNormPath::kPersistent;
    const PersistentCfg* pc = nullptr;
    switch (mode) {
      case Norm::kRms: pc = pick_persistent(kRmsPersistent, nchunk, args.M, forced); break;
      case Norm::kLayer: pc = pick_persistent(kLayerPersistent, nchunk, args.M, forced); break;
      case Norm::kL2: pc = pick_persistent(kL2Persistent, nchunk, args.M, forced); break;
      case Norm::kAddRms: break;
    }
    if (forced && !pc) return hipErrorInvalidValue;
    if (pc) {
      const int64_t sets = (args.M + pc->rpl - 1) / pc->rpl;
      int64_t g = grid > 0 ? grid : pc->grid;
      if (g > sets) g = sets;
      const RowNormKernel kernel = (nchunk == 64 * pc->wpr * pc->maxc) ? pc->full[d] : pc->ragged[d];
      return dispatch(kernel, dim3((unsigned)g), dim3(64 * pc->wpr), persistent_lds_bytes(*pc, nchunk),
                      stream, args);
    }
  }

  if (!cfg) return hipErrorInvalidValue;
  if (cfg->wpr > 1 && nchunk < 64 * cfg->wpr) return hipErrorInvalidValue;  // table invariant
  const int rows_per_wg = cfg->rows * cfg->rpl;
  const int threads = 64 * cfg->wpr * cfg->rows;
  const size_t lds = cfg->regs ? rownorm_regs_lds_bytes(cfg->wgs_per_cu)
                                : rownorm_lds_bytes(rows_per_wg, N, cfg->wgs_per_cu);
  if (nchunk > cfg->full_nchunk) return hipErrorInvalidValue;  // table invariant
  const int64_t all_blocks = (args.M + rows_per_wg - 1) / rows_per_wg;
  const RowNormKernel kernel = nchunk != cfg->full_nchunk ? cfg->ragged[d]
                               : cfg->full_cw[d] && all_blocks >= kChunkWaitMinBlocks ? cfg->full_cw[d]
                                                                                      : cfg->full[d];
  if (!kernel) return hipErrorInvalidValue;  // table invariant (exact _R entries have no ragged kernel)
  args.xcd_group = cfg->xcd_group;
  // One dispatch covers at most kMaxWorkItems work-items: larger launches run
  // as several launches over consecutive row ranges (rows are independent).
  const int64_t rows_per_launch = (kMaxWorkItems / threads) * rows_per_wg;
  for (int64_t r0 = 0; r0 < args.M; r0 += rows_per_launch) {
    RowNormArgs part = args;
    const int64_t e0 = r0 * N;
    part.x = args.x + e0;
    part.y = args.y + e0;
    if (args.r) part.r = args.r + e0;
    if (args.h) part.h = args.h + e0;
    part.M = args.M - r0 < rows_per_launch ? args.M - r0 : rows_per_launch;
    const int64_t blocks = (part.M + rows_per_wg - 1) / rows_per_wg;
    const hipError_t err = dispatch(kernel, dim3((unsigned)blocks), dim3(threads), lds, stream, part);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace mbn
