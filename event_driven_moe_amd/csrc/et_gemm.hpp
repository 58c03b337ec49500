// et_gemm.hpp -- bf16 MFMA tiles for the GEMM tasks (gfx950, wave64).
//
// Both tiles accumulate in fp32 with v_mfma_f32_16x16x32_bf16 and take the
// weights (B) K-contiguous ([N, K]) straight from global memory into VGPRs in
// MFMA operand layout: lane (j = lane%16, g = lane/16) of a 16-column group
// holds column j.  For one 128-element K-block, the s-th of four 16-byte
// loads takes chunk 4s + g of the row's 256 bytes, so one load instruction
// covers 64 contiguous bytes of each of its 16 rows (16 memory sectors for
// 1 KB; with the chunks of a lane group adjacent instead, one instruction
// touched 64 sectors and the streaming rate per CU was a quarter as high),
// and the four loads together read whole cache lines of the weight stream.
// MFMA step s (0..3) consumes elements 32s + 8g .. 32s + 8g + 7 of both
// operands, the MFMA's natural K order.
//
// StreamTile (few rows, the decode regime): A also streams from global memory
// into VGPRs (lane (i = lane%16, g) holds row i).  The four waves split the
// tile as WK (K-split) x 4/WK (N-split); with WK > 1 wave wk consumes K-blocks
// wk, wk + WK, ... and the partial tiles are summed through LDS.  Loads run PD
// K-blocks ahead of the MFMAs (a register ring), keeping enough bytes in
// flight per CU to stream weights at HBM rate.
//
// RingTile (many rows, the MFMA-bound regime): 16*MT rows x 256 columns, the
// four waves splitting the columns (64 each, four 16-column groups).  Both
// operands of a 64-element K-stage are copied straight from global memory
// into LDS by the buffer unit (16 bytes per lane, no VGPR staging), into a
// ring of three stages, so two stages are always in flight while the MFMAs
// consume the third.  Rows are 128 bytes with the 16-byte chunks XOR-swizzled
// by (row / 2) mod 8: the copy writes whole rows contiguously and the 16
// rows one ds_read_b128 reads fall into 16 disjoint 4-bank groups.
//
// In both, rows outside the valid range use an out-of-range buffer offset and
// read as zeros, and A can be read agent-coherently (COH) when it was written
// earlier in the same launch.  gate(round) runs uniformly on all waves before
// the A loads of a round (gate(0) always runs and may fill the row table); the
// weights of the first rounds are requested before gate(0), so the weight
// stream starts before the activations it multiplies are ready (the prefetch
// rewrite of Event Tensor notes, section "ETC 编译流程", and the weight
// prefetch of section "端到端低 batch serving").
#pragma once

#include "et_device.hpp"

namespace et {

template <int MT, int NB, int WK, int PD, bool COH>
struct StreamTile {
  static constexpr int kRedFloats = WK > 1 ? 4 * MT * NB * 4 * 64 : 1;   // LDS floats
  static constexpr int kLdsBytes = kRedFloats * 4;   // reduction scratch
  static constexpr int kStageBytes = 0;                // no LDS ring

  // acc[mt][nb]: rows 16*mt + 4*(lane/16) + r, column 16*nb + lane%16 of this
  // wave's column group (for WK > 1: summed over the K-split waves).
  f32x4 acc[MT][NB];

  template <class Gate>
  __device__ __forceinline__ bool run(Rsrc ra, const uint32_t* a_row_off /* [16*MT], LDS */,
                                      const Rsrc* rb, const uint32_t* b_row_off /* [NB] */,
                                      int nkb, Gate gate, float* red /* LDS kRedFloats */) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar registers
    const int wk = wave % WK;
    const uint32_t kg = (uint32_t)(lane >> 4) * 16u;   // chunk 4 s + g of a K-block row
    uint32_t aoff[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int n = 0; n < NB; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int rounds = (nkb + WK - 1) / WK;
    i32x4 abuf[PD][MT][4];
    i32x4 bbuf[PD][NB][4];

    auto load_b = [&](int p, int round) {
      const int kb = round * WK + wk;
      if (round < rounds && kb < nkb) {
        const uint32_t o = (uint32_t)kb * 256u + kg;
#pragma unroll
        for (int n = 0; n < NB; ++n)
#pragma unroll
          for (int s = 0; s < 4; ++s) bbuf[p][n][s] = ld16(rb[n], b_row_off[n] + o + 64u * s);
      }
    };
    auto load_a = [&](int p, int round) {
      const int kb = round * WK + wk;
      if (round < rounds && kb < nkb) {
        const uint32_t o = (uint32_t)kb * 256u + kg;
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int s = 0; s < 4; ++s) abuf[p][m][s] = ld16x<COH>(ra, aoff[m] + o + 64u * s);
      }
    };

#pragma unroll
    for (int p = 0; p < PD; ++p) load_b(p, p);
    if (!gate(0)) return false;
#pragma unroll
    for (int m = 0; m < MT; ++m) aoff[m] = a_row_off[16 * m + (lane & 15)];
    load_a(0, 0);
#pragma unroll
    for (int p = 1; p < PD; ++p) {
      if (p < rounds && !gate(p)) return false;
      load_a(p, p);
    }

    for (int j = 0; j < rounds; j += PD) {
#pragma unroll
      for (int p = 0; p < PD; ++p) {
        const int round = j + p;
        const int kb = round * WK + wk;
        if (round < rounds && kb < nkb) {
#pragma unroll
          for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
              for (int n = 0; n < NB; ++n) acc[m][n] = mfma16(abuf[p][m][s], bbuf[p][n][s], acc[m][n]);
        }
        const int nxt = round + PD;
        load_b(p, nxt);
        if (nxt < rounds && !gate(nxt)) return false;
        load_a(p, nxt);
      }
    }

    if (WK > 1) {
      const int wn = wave / WK;
      __syncthreads();
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int n = 0; n < NB; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r) red[(((wave * MT + m) * NB + n) * 4 + r) * 64 + lane] = acc[m][n][r];
      __syncthreads();
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int n = 0; n < NB; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float v = 0.f;
#pragma unroll
            for (int q = 0; q < WK; ++q) v += red[((((wn * WK + q) * MT + m) * NB + n) * 4 + r) * 64 + lane];
            acc[m][n][r] = v;
          }
      __syncthreads();
    }
    return true;
  }
};

// 16 bytes per lane, global -> LDS at lds_base + 16 * lane (sc1 when COH).
// Issued from inline asm: the compiler's own wait insertion cannot tell the
// ring slots' copies apart and would drain every copy in flight before each
// LDS read; the tiles order the copies themselves with explicit vmcnt waits
// and barriers.  M0 (the LDS base of the copy) is restored afterwards.
template <bool COH>
__device__ __forceinline__ void dma16(Rsrc r, void* lds_base, uint32_t voff) {
  const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  uint32_t save;
  if constexpr (COH)
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                 "buffer_load_dwordx4 %2, %3, 0 offen sc1 lds\n\ts_mov_b32 m0, %0"
                 : "=&s"(save) : "s"(l), "v"(voff), "s"(r) : "memory");
  else
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                 "buffer_load_dwordx4 %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
                 : "=&s"(save) : "s"(l), "v"(voff), "s"(r) : "memory");
}

// Workgroup barrier that waits for this wave's LDS accesses only (the
// compiler's __syncthreads also waits for every outstanding global store).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until at most N of this wave's memory loads are outstanding, then the
// workgroup barrier (a compiler memory barrier too).
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"i"(N) : "memory");
}

template <int MT, bool COH>
struct RingTile {
  static constexpr int kRows = 16 * MT;                   // A rows
  static constexpr int kCols = 256;                       // B rows = output columns
  static constexpr int kStageBytes = (kRows + kCols) * 128;
  static constexpr int kLdsBytes = 0;                     // besides the three ring slots
  static constexpr int kLA = kRows / 32;                  // A copies per wave per stage
  static constexpr int kLB = 8;                           // B copies per wave per stage
  static constexpr int kL = kLA + kLB;

  f32x4 acc[MT][4];

  // fragment i of a K-step (i < 4: B group i of this wave, else A group i-4)
  __device__ static __forceinline__ i32x4 frag(const unsigned char* slot, uint32_t fo, int wave, int i) {
    const unsigned char* p = i < 4 ? slot + kRows * 128 + wave * 64 * 128 + i * 16 * 128
                                   : slot + (i - 4) * 16 * 128;
    return *reinterpret_cast<const i32x4*>(p + fo);
  }

  // One K-step over the valid 16-row groups (2 * NV of them): the MFMAs on
  // (af, bf), two per group, fenced so that the next K-step's fragment reads
  // (READ) and the copies dma(0..) of a later stage (DMA) sit between them.
  // The next B fragments go to nbf; the next A fragments replace af[m] as
  // soon as the MFMAs of row pair m have been issued.
  template <int NV, bool READ, bool DMA, class DmaF>
  __device__ __forceinline__ void kstep(i32x4* af, const i32x4* bf, const unsigned char* rslot,
                                        uint32_t fo, int wave, i32x4* nbf, DmaF dma) {
    constexpr int kNG = 4 * NV;                 // groups of two MFMAs
    constexpr int kND = kLB + NV;               // copies (A copies of valid halves only)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < kNG; ++g) {
      const int m = 2 * (g / 4), n = g % 4;
      acc[m][n] = mfma16(af[m], bf[n], acc[m][n]);
      acc[m + 1][n] = mfma16(af[m + 1], bf[n], acc[m + 1][n]);
      if constexpr (READ) {
        if (g < 4) nbf[g] = frag(rslot, fo, wave, g);
        if (n == 3) {
          af[m] = frag(rslot, fo, wave, 4 + m);
          af[m + 1] = frag(rslot, fo, wave, 5 + m);
        }
      }
      if constexpr (DMA) {
#pragma unroll
        for (int i = g * kND / kNG; i < (g + 1) * kND / kNG; ++i) dma(i);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // rb[n] / b_row0[n]: buffer and byte offset of the first row (output
  // column) of this wave's 16-column group n; rows are b_stride bytes apart.
  // s0, s1, s2: the three ring slots, kStageBytes each.
  // mv: 16-row groups holding valid rows (1..MT); 32-row halves beyond them
  // are neither copied nor multiplied (their rows would read as zeros and
  // their results are not stored).
  template <class Gate>
  __device__ __forceinline__ bool run(Rsrc ra, const uint32_t* a_row_off /* [kRows], LDS */,
                                      const Rsrc* rb, const uint32_t* b_row0, uint32_t b_stride,
                                      int K, Gate gate, unsigned char* s0, unsigned char* s1,
                                      unsigned char* s2, int mv = MT) {
    const int nv = (min(max(mv, 1), MT) + 1) >> 1;    // valid 32-row halves
    if constexpr (MT >= 8) {
      if (nv == 4) return body<4>(ra, a_row_off, rb, b_row0, b_stride, K, gate, s0, s1, s2);
      if (nv == 3) return body<3>(ra, a_row_off, rb, b_row0, b_stride, K, gate, s0, s1, s2);
    }
    if constexpr (MT >= 4)
      if (nv == 2) return body<2>(ra, a_row_off, rb, b_row0, b_stride, K, gate, s0, s1, s2);
    return body<1>(ra, a_row_off, rb, b_row0, b_stride, K, gate, s0, s1, s2);
  }

  // Software pipeline over 64-element K-stages held in a ring of three LDS
  // slots, all three in flight ahead of the MFMAs.  Per stage ks (slot cur):
  // K-step 0 multiplies fragments already in VGPRs while reading K-step 1's;
  // then the wait for stage ks+1 (this wave's copies, then the barrier for
  // everyone's -- which also tells that every wave is done reading slot cur);
  // K-step 1 multiplies while stage ks+1's first fragments are read and
  // stage ks+3 is copied into slot cur.
  template <int NV, class Gate>
  __device__ __forceinline__ bool body(Rsrc ra, const uint32_t* a_row_off, const Rsrc* rb,
                                       const uint32_t* b_row0, uint32_t b_stride, int K, Gate gate,
                                       unsigned char* s0, unsigned char* s1, unsigned char* s2) {
    constexpr int kLAv = NV;                    // A copies per wave per stage (valid halves)
    constexpr int kLv = kLB + kLAv;
    constexpr int kNR = 4 + 2 * NV;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar registers
    const int nks = K / 64;
    const int crow = lane >> 3, cpos = lane & 7;   // this lane's row / chunk in a copy
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int n = 0; n < 4; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

    // B copies: wave-local rows 8q + crow (group q / 2); the logical chunk of
    // this lane's physical slot cpos is cpos ^ ((row / 2) mod 8)
    uint32_t boff[kLB];
#pragma unroll
    for (int q = 0; q < kLB; ++q) {
      const int j = 8 * (q & 1) + crow;
      const int c = cpos ^ ((j >> 1) & 7);
      boff[q] = b_row0[q >> 1] + (uint32_t)j * b_stride + 16u * c;
    }
    uint32_t aoff[kLAv];
    // copy i of stage ks into slot: i < kLB weight rows, else A half i - kLB
    auto dma_one = [&](int i, int ks, unsigned char* slot) ET_INLINE {
      if (i < kLB)
        dma16<false>(rb[i >> 1], slot + kRows * 128 + wave * 64 * 128 + i * 1024, boff[i] + ks * 128u);
      else
        dma16<COH>(ra, slot + (wave + 4 * (i - kLB)) * 1024, aoff[i - kLB] + ks * 128u);
    };

    // the weights of the first stages are requested before the gate
#pragma unroll
    for (int q = 0; q < kLB; ++q) dma_one(q, 0, s0);
    if (nks > 1)
#pragma unroll
      for (int q = 0; q < kLB; ++q) dma_one(q, 1, s1);
    if (nks > 2)
#pragma unroll
      for (int q = 0; q < kLB; ++q) dma_one(q, 2, s2);
    if (!gate(0)) {
      wait_vm_barrier<0>();
      return false;
    }
#pragma unroll
    for (int u = 0; u < kLAv; ++u) {
      const int row = 8 * (wave + 4 * u) + crow;
      const uint32_t base = a_row_off[row];
      aoff[u] = base == kOOB ? kOOB : base + 16u * (uint32_t)(cpos ^ ((row >> 1) & 7));
    }
#pragma unroll
    for (int u = 0; u < kLAv; ++u) dma_one(kLB + u, 0, s0);
    if (nks > 1)
#pragma unroll
      for (int u = 0; u < kLAv; ++u) dma_one(kLB + u, 1, s1);
    if (nks > 2)
#pragma unroll
      for (int u = 0; u < kLAv; ++u) dma_one(kLB + u, 2, s2);

    // fragment read offsets: row (lane % 16) of each 16-row group, logical
    // chunk 4h + g -> physical chunk (4h + g) ^ ((lane % 16) / 2 mod 8)
    const int fi = lane & 15, fg = lane >> 4;
    uint32_t foff[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      foff[h] = (uint32_t)fi * 128u + 16u * (uint32_t)((4 * h + fg) ^ ((fi >> 1) & 7));

    // stage 0 complete: only the A copies of stages 1 and 2 were issued after it
    if (nks > 2) wait_vm_barrier<2 * kLAv>();
    else if (nks > 1) wait_vm_barrier<kLAv>();
    else wait_vm_barrier<0>();
    i32x4 fa[MT], fb0[4], fb1[4];
#pragma unroll
    for (int i = 0; i < kNR; ++i) {
      if (i < 4) fb0[i] = frag(s0, foff[0], wave, i);
      else fa[i - 4] = frag(s0, foff[0], wave, i);
    }
    auto no_dma = [](int) {};
    // slot of stage ks: ring position ks mod 3 (rotated at run time, so the
    // steady-state stage is one copy of code)
    unsigned char* cur = s0;
    unsigned char* nxt = s1;
    unsigned char* nx2 = s2;
    auto rotate = [&]() ET_INLINE {
      unsigned char* t = cur;
      cur = nxt;
      nxt = nx2;
      nx2 = t;
    };
    // stage 1's wait: after it only stage 2's A copies were issued; later
    // stages wait with stage ks+2 (all of its copies) still in flight
    auto wait_next = [&](int ks) ET_INLINE {
      if (ks == 0) wait_vm_barrier<kLAv>();
      else wait_vm_barrier<kLv>();
    };
    int ks = 0;
    for (; ks + 3 < nks; ++ks) {            // steady state: stage ks+3 is copied into slot cur
      kstep<NV, true, false>(fa, fb0, cur, foff[1], wave, fb1, no_dma);
      wait_next(ks);
      unsigned char* dst = cur;
      const int kd = ks + 3;
      kstep<NV, true, true>(fa, fb1, nxt, foff[0], wave, fb0,
                            [&](int i) ET_INLINE { dma_one(i, kd, dst); });
      rotate();
    }
    for (; ks < nks; ++ks) {                // the last (up to) three stages
      kstep<NV, true, false>(fa, fb0, cur, foff[1], wave, fb1, no_dma);
      if (ks + 1 < nks) {
        if (ks + 2 < nks) wait_next(ks);
        else wait_vm_barrier<0>();
        kstep<NV, true, false>(fa, fb1, nxt, foff[0], wave, fb0, no_dma);
      } else {
        kstep<NV, false, false>(fa, fb1, nxt, foff[0], wave, fb0, no_dma);
      }
      rotate();
    }
    wait_vm_barrier<0>();            // the ring may be refilled by the next task
    return true;
  }
};

}  // namespace et
