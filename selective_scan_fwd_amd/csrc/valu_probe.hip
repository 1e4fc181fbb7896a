// Issue-rate probe for the vector ALU forms that the scan's state step is
// made of (gfx950).  It backs the ALU roofline that the benchmark prices the
// scan against: how many SIMD cycles a wave64 instruction of each form takes
// when the SIMD has enough independent work, and what the scan's own
// instruction mix costs per state update.
//
// Each probe kernel runs `iters` iterations of a fixed, fully unrolled body on
// every wave, with no memory traffic inside the loop.  Lane 0 of every wave
// records the shader-clock counter (s_memtime) and the 100 MHz real-time
// counter (s_memrealtime) around the loop; the host divides a wave's elapsed
// shader cycles by the wave-instructions its SIMD issued meanwhile.
//
// Bodies (instruction counts per iteration are the ones the disassembly of
// this file shows; kProbeInstr holds them):
//   0 fma      16 independent chains of v_fma_f32
//   1 exp      16 independent chains of v_exp_f32 (x <- 2^-x, which settles
//              near 0.64, so every operand stays a normal number)
//   2 mix      1 v_exp_f32 per 4 v_fma_f32, all chains independent
//   3 state    the scan's step for one lane: 8 steps x 4 states of
//              dA = 2^(dt a), h = dA h + dtu * bcast(B), y += bcast(C) h,
//              B and C taken through DPP row broadcasts as in the scan
//   4 state-noexp  the same with v_exp_f32 replaced by a v_mul_f32
//   5 permlane 16 independent v_permlane32_swap_b32 exchanges
//   6 exp-latency  one dependent chain of v_exp_f32 (one wave per SIMD)
//   7 fma-latency  one dependent chain of v_fma_f32
//   8-12  operand forms (three VGPRs, two VGPRs, an SGPR, v_fmac with an
//         SGPR, a DPP row broadcast); 13-14 the state step with B and C in
//         SGPRs (one lane per channel), with and without the exponential;
//   15    exp waves and fma waves sharing each SIMD; 16-17 the state step
//         with every operand in VGPRs; 18-21 the state step in
//         barrier-separated exponential and non-exponential phases (2 or 4
//         waves per SIMD from one workgroup; with and without the barrier)
//   22-23 instruction fetch: 4096 fma as straight-line code run once, or as
//         a loop of 64
//   24-26 the state step with every operand in VGPRs (as 16), its
//         exponentials grouped per wave: each iteration first takes the
//         exponentials of 1, 2 or 4 steps (16, 32 or 64 in a row), then the
//         writes, state updates and readouts of those steps; no barrier, so
//         the waves sharing a SIMD drift in and out of phase
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ float opaque(float v) {
  asm volatile("" : "+v"(v));
  return v;
}

template <int J>
__device__ __forceinline__ float row_bcast(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + J, 0xf, 0xf, true));
}

template <int J> __device__ __forceinline__ void fmac_bcast(float &y, float c, float h);
#define PROBE_FMAC(J)                                                                  \
  template <>                                                                          \
  __device__ __forceinline__ void fmac_bcast<J>(float &y, float c, float h) {          \
    asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:" #J " row_mask:0xf bank_mask:0xf"     \
        : "+v"(y)                                                                      \
        : "v"(c), "v"(h));                                                             \
  }
PROBE_FMAC(5) PROBE_FMAC(6) PROBE_FMAC(7)
#undef PROBE_FMAC

template <bool EXP>
__device__ __forceinline__ void state4(float (&h)[4], const float (&a2)[4], float dt, float dtu,
                                       float bc, float &y) {
  float dA = EXP ? __builtin_amdgcn_exp2f(dt * a2[0]) : (dt * a2[0]) * 0.5f;
  h[0] = __builtin_fmaf(dA, h[0], dtu * row_bcast<0>(bc));
  y = row_bcast<4>(bc) * h[0];
  dA = EXP ? __builtin_amdgcn_exp2f(dt * a2[1]) : (dt * a2[1]) * 0.5f;
  h[1] = __builtin_fmaf(dA, h[1], dtu * row_bcast<1>(bc));
  fmac_bcast<5>(y, bc, h[1]);
  dA = EXP ? __builtin_amdgcn_exp2f(dt * a2[2]) : (dt * a2[2]) * 0.5f;
  h[2] = __builtin_fmaf(dA, h[2], dtu * row_bcast<2>(bc));
  fmac_bcast<6>(y, bc, h[2]);
  dA = EXP ? __builtin_amdgcn_exp2f(dt * a2[3]) : (dt * a2[3]) * 0.5f;
  h[3] = __builtin_fmaf(dA, h[3], dtu * row_bcast<3>(bc));
  fmac_bcast<7>(y, bc, h[3]);
}

// Workgroup size and dynamic LDS of each body: the phased bodies run one
// workgroup per CU (8 or 16 waves: 2 or 4 per SIMD, 96 KB of LDS each).
constexpr int probe_threads(int kind) { return kind == 18 || kind == 19 ? 512 : kind == 20 || kind == 21 ? 1024 : 256; }
constexpr int probe_lds(int kind) { return kind >= 18 && kind <= 21 ? 96 * 1024 : 0; }

template <int KIND>
__global__ void __launch_bounds__(probe_threads(KIND)) probe_kernel(const float *in, float *out, uint64_t *clk, int iters) {
  const int lane = threadIdx.x & 63;
  const int tid = blockIdx.x * blockDim.x + threadIdx.x;
  const float s = in[lane];
  float acc = 0.0f;
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  if constexpr (KIND == 0 || KIND == 1 || KIND == 2) {
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = s + 0.01f * i;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int rep = 0; rep < 4; ++rep) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if (KIND == 0 || (KIND == 2 && (i & 3) != 0)) x[i] = __builtin_fmaf(x[i], 0.999f, 0.001f);
          else x[i] = __builtin_amdgcn_exp2f(-x[i]);
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = opaque(x[i]);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) acc += x[i];
  } else if constexpr (KIND == 3 || KIND == 4) {
    float h[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    float a2[4], dt[8], dtu[8], bc[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) a2[j] = opaque(-(j + 1) * 1.4426950408889634f);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      dt[q] = 0.01f + 0.001f * q;
      dtu[q] = s * dt[q];
      bc[q] = in[(lane + q) & 63];
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        dt[q] = opaque(dt[q]);
        dtu[q] = opaque(dtu[q]);
        bc[q] = opaque(bc[q]);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        float y;
        state4<KIND == 3>(h, a2, dt[q], dtu[q], bc[q], y);
        acc += y;
      }
    }
    acc += h[0] + h[1] + h[2] + h[3];
  } else if constexpr (KIND == 5) {
    uint32_t v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = __builtin_bit_cast(uint32_t, s) + i;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int rep = 0; rep < 4; ++rep) {
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          auto r = __builtin_amdgcn_permlane32_swap(v[i], v[i + 1], false, false);
          v[i] = r[0];
          v[i + 1] = r[1];
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = __builtin_bit_cast(uint32_t, opaque(__builtin_bit_cast(float, v[i])));
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) acc += __builtin_bit_cast(float, v[i]);
  } else if constexpr (KIND >= 8 && KIND <= 12) {
    // operand forms: 16 independent chains, 64 instructions per iteration
    float x[16], y[16], zz[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      x[i] = s + 0.01f * i;
      y[i] = opaque(0.999f - 0.001f * i);
      zz[i] = opaque(0.001f * i);
    }
    float sc = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, in[48])));
    for (int it = 0; it < iters; ++it) {
      asm volatile("" : "+s"(sc));
#pragma unroll
      for (int rep = 0; rep < 4; ++rep) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if constexpr (KIND == 8) x[i] = __builtin_fmaf(x[i], y[i], zz[i]);   // three VGPRs
          else if constexpr (KIND == 9) x[i] = x[i] * y[i];                    // two VGPRs
          else if constexpr (KIND == 10) x[i] = x[i] * sc;                     // SGPR operand
          else if constexpr (KIND == 11) x[i] = __builtin_fmaf(sc, y[i], x[i]); // v_fmac with SGPR
          else                                                                  // DPP row broadcast
            asm("v_mul_f32_dpp %0, %1, %0 row_newbcast:1 row_mask:0xf bank_mask:0xf" : "+v"(x[i]) : "v"(y[i]));
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = opaque(x[i]);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) acc += x[i];
  } else if constexpr (KIND == 13 || KIND == 14) {
    // one lane owns all 16 states of its channel; B and C of the step are
    // wave-uniform scalars: dA = 2^(dt a), h = dA h + dtu B, y += C h
    float h[16], a2[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      h[j] = 0.0f;
      a2[j] = opaque(-(j + 1) * 1.4426950408889634f);
    }
    float bs[16], cs[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      bs[j] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, in[j])));
      cs[j] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, in[16 + j])));
    }
    float dt = 0.01f + 0.0001f * lane, dtu = s * dt;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        dt = opaque(dt);
        dtu = opaque(dtu);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          asm volatile("" : "+s"(bs[j]));
          asm volatile("" : "+s"(cs[j]));
        }
        float y = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float dA = KIND == 13 ? __builtin_amdgcn_exp2f(dt * a2[j]) : (dt * a2[j]) * 0.5f;
          h[j] = __builtin_fmaf(dA, h[j], dtu * bs[j]);
          y = __builtin_fmaf(cs[j], h[j], y);
        }
        acc += y;
      }
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) acc += h[j];
  } else if constexpr (KIND == 15) {
    // exp waves: 16 exp chains; fma waves: 16 fma chains (a separate
    // transcendental pipe would let the two kinds of wave overlap)
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = s + 0.01f * i;
    // workgroups are dispatched round-robin over the 256 CUs: workgroups
    // 256 k .. 256 k + 255 form one round, so alternating rounds put one
    // exp wave and one fma wave on every SIMD
    const bool ewave = ((blockIdx.x >> 8) & 1) != 0;
    if (ewave) {
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int rep = 0; rep < 4; ++rep)
#pragma unroll
          for (int i = 0; i < 16; ++i) x[i] = __builtin_amdgcn_exp2f(-x[i]);
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = opaque(x[i]);
      }
    } else {
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int rep = 0; rep < 4; ++rep)
#pragma unroll
          for (int i = 0; i < 16; ++i) x[i] = __builtin_fmaf(x[i], 0.999f, 0.001f);
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = opaque(x[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) acc += x[i];
  } else if constexpr (KIND == 16 || KIND == 17) {
    // one lane owns 16 states; B and C of the step are uniform values held
    // in VGPRs (every operand a VGPR)
    float h[16], a2[16], bv[16], cv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      h[j] = 0.0f;
      a2[j] = opaque(-(j + 1) * 1.4426950408889634f);
      bv[j] = opaque(in[j]);
      cv[j] = opaque(in[16 + j]);
    }
    float dt = 0.01f + 0.0001f * lane, dtu = s * dt;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        dt = opaque(dt);
        dtu = opaque(dtu);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          bv[j] = opaque(bv[j]);
          cv[j] = opaque(cv[j]);
        }
        float y = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float dA = KIND == 16 ? __builtin_amdgcn_exp2f(dt * a2[j]) : (dt * a2[j]) * 0.5f;
          h[j] = __builtin_fmaf(dA, h[j], dtu * bv[j]);
          y = __builtin_fmaf(cv[j], h[j], y);
        }
        acc += y;
      }
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) acc += h[j];
  } else if constexpr (KIND >= 18 && KIND <= 21) {
    // Phased state step: 16 states per lane, 4 steps per phase.  Phase A
    // takes the 64 exponentials of the tile, phase B every other operation
    // (write, state update, readout and the next tile's exponents).  With
    // SYNC the waves of the workgroup (all the waves of the CU: the launch
    // reserves most of its LDS) meet at a barrier between the phases, so
    // the waves sharing a SIMD run the same phase together.
    constexpr bool SYNC = KIND == 18 || KIND == 20;
    float h[16], a2[16], e[4][16], dt[4], dtu[4];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      h[j] = 0.0f;
      a2[j] = opaque(-(j + 1) * 1.4426950408889634f);
    }
    float bs[16], cs[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      bs[j] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, in[j])));
      cs[j] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, in[16 + j])));
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      dt[q] = 0.01f + 0.0001f * (lane + q);
      dtu[q] = s * dt[q];
#pragma unroll
      for (int j = 0; j < 16; ++j) e[q][j] = dt[q] * a2[j];
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < 16; ++j) e[q][j] = __builtin_amdgcn_exp2f(e[q][j]);
      __builtin_amdgcn_sched_barrier(0);     // the compiler keeps the phases apart
      if constexpr (SYNC) __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        asm volatile("" : "+s"(bs[j]));
        asm volatile("" : "+s"(cs[j]));
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        dt[q] = opaque(dt[q]);
        dtu[q] = opaque(dtu[q]);
        float y = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          h[j] = __builtin_fmaf(e[q][j], h[j], dtu[q] * bs[j]);
          y = __builtin_fmaf(cs[j], h[j], y);
          e[q][j] = dt[q] * a2[j];
        }
        acc += y;
      }
      __builtin_amdgcn_sched_barrier(0);     // the compiler keeps the phases apart
      if constexpr (SYNC) __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) acc += h[j];
  } else if constexpr (KIND >= 24 && KIND <= 26) {
    constexpr int QS = KIND == 24 ? 1 : KIND == 25 ? 2 : 4;   // steps per group
    float h[16], a2[16], bv[16], cv[16], e[QS][16], dt[QS], dtu[QS];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      h[j] = 0.0f;
      a2[j] = opaque(-(j + 1) * 1.4426950408889634f);
      bv[j] = opaque(in[j]);
      cv[j] = opaque(in[16 + j]);
    }
#pragma unroll
    for (int q = 0; q < QS; ++q) {
      dt[q] = 0.01f + 0.0001f * (lane + q);
      dtu[q] = s * dt[q];
#pragma unroll
      for (int j = 0; j < 16; ++j) e[q][j] = dt[q] * a2[j];
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int q = 0; q < QS; ++q)
#pragma unroll
        for (int j = 0; j < 16; ++j) e[q][j] = __builtin_amdgcn_exp2f(e[q][j]);
      __builtin_amdgcn_sched_barrier(0);     // the compiler keeps the groups apart
#pragma unroll
      for (int q = 0; q < QS; ++q) {
        dt[q] = opaque(dt[q]);
        dtu[q] = opaque(dtu[q]);
        float y = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          h[j] = __builtin_fmaf(e[q][j], h[j], dtu[q] * bv[j]);
          y = __builtin_fmaf(cv[j], h[j], y);
          e[q][j] = dt[q] * a2[j];
        }
        acc += y;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) acc += h[j];
  } else if constexpr (KIND == 22 || KIND == 23) {
    // instruction fetch: 4096 independent v_fma_f32 as straight-line code
    // run once (22), or as 64 passes of a 64-instruction loop (23)
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = s + 0.01f * i;
    for (int it = 0; it < iters; ++it) {
      if constexpr (KIND == 22) {
#pragma unroll
        for (int rep = 0; rep < 256; ++rep)
#pragma unroll
          for (int i = 0; i < 16; ++i) x[i] = __builtin_fmaf(x[i], 0.999f + 1e-7f * rep, 0.001f);
      } else {
#pragma unroll
        for (int rep = 0; rep < 4; ++rep)
#pragma unroll
          for (int i = 0; i < 16; ++i) x[i] = __builtin_fmaf(x[i], 0.999f + 1e-7f * rep, 0.001f);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = opaque(x[i]);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) acc += x[i];
  } else {
    float x = s;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int rep = 0; rep < 64; ++rep)
        x = KIND == 6 ? __builtin_amdgcn_exp2f(-x) : __builtin_fmaf(x, 0.999f, 0.001f);
      x = opaque(x);
    }
    acc = x;
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  out[tid] = acc;
  if (lane == 0) {
    const int w = tid >> 6;
    clk[4 * w + 0] = t0;
    clk[4 * w + 1] = t1;
    clk[4 * w + 2] = r0;
    clk[4 * w + 3] = r1;
  }
}


template <int KIND>
hipError_t launch(int blocks, int iters, const float *in, float *out, uint64_t *clk, hipStream_t st) {
  if (probe_lds(KIND) > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(probe_kernel<KIND>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, probe_lds(KIND));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(probe_kernel<KIND>, dim3(blocks), dim3(probe_threads(KIND)), probe_lds(KIND), st, in, out,
                     clk, iters);
  return hipGetLastError();
}

}  // namespace

extern "C" {

// Wave-instructions per iteration of each body, as in its disassembly
// (loop control excluded): VALU forms only.
const int kProbeInstr[27] = {64, 64, 64, 168, 168, 32, 64, 64, 64, 64, 64, 64, 64, 162, 162, 64, 162, 162,
                             324, 324, 324, 324, 4096, 64, 97, 162, 324};

// Runs probe `kind` on `blocks` workgroups of vm_probe_threads(kind)
// threads for `iters` iterations.  in: 64 floats (device); out: blocks *
// threads floats (device); clk: blocks * threads / 64 * 4 uint64 (device;
// per wave: shader clock start and end, real-time start and end).  Returns a hipError_t value (0 = success).
int vm_probe_run(int kind, int blocks, int iters, const void *in, void *out, void *clk, void *stream) {
  if (blocks <= 0 || iters <= 0 || in == nullptr || out == nullptr || clk == nullptr) return 1;
  const float *i = static_cast<const float *>(in);
  float *o = static_cast<float *>(out);
  uint64_t *c = static_cast<uint64_t *>(clk);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (kind) {
    case 0: return launch<0>(blocks, iters, i, o, c, s);
    case 1: return launch<1>(blocks, iters, i, o, c, s);
    case 2: return launch<2>(blocks, iters, i, o, c, s);
    case 3: return launch<3>(blocks, iters, i, o, c, s);
    case 4: return launch<4>(blocks, iters, i, o, c, s);
    case 5: return launch<5>(blocks, iters, i, o, c, s);
    case 6: return launch<6>(blocks, iters, i, o, c, s);
    case 7: return launch<7>(blocks, iters, i, o, c, s);
    case 8: return launch<8>(blocks, iters, i, o, c, s);
    case 9: return launch<9>(blocks, iters, i, o, c, s);
    case 10: return launch<10>(blocks, iters, i, o, c, s);
    case 11: return launch<11>(blocks, iters, i, o, c, s);
    case 12: return launch<12>(blocks, iters, i, o, c, s);
    case 13: return launch<13>(blocks, iters, i, o, c, s);
    case 14: return launch<14>(blocks, iters, i, o, c, s);
    case 15: return launch<15>(blocks, iters, i, o, c, s);
    case 16: return launch<16>(blocks, iters, i, o, c, s);
    case 17: return launch<17>(blocks, iters, i, o, c, s);
    case 18: return launch<18>(blocks, iters, i, o, c, s);
    case 19: return launch<19>(blocks, iters, i, o, c, s);
    case 20: return launch<20>(blocks, iters, i, o, c, s);
    case 21: return launch<21>(blocks, iters, i, o, c, s);
    case 22: return launch<22>(blocks, iters, i, o, c, s);
    case 23: return launch<23>(blocks, iters, i, o, c, s);
    case 24: return launch<24>(blocks, iters, i, o, c, s);
    case 25: return launch<25>(blocks, iters, i, o, c, s);
    case 26: return launch<26>(blocks, iters, i, o, c, s);
    default: return 1;
  }
}

int vm_probe_instr(int kind) { return kind >= 0 && kind < 27 ? kProbeInstr[kind] : 0; }
int vm_probe_threads(int kind) { return probe_threads(kind); }

}  // extern "C"
