/*
 * Roofline probes for MI355X (gfx950): the achievable HBM bandwidth, bf16
 * matrix-core rate and vector-ALU issue rate of the machine they run on, measured beside the path's
 * own kernels so that each kernel can be placed against what the hardware
 * delivers as well as against the datasheet peaks (HBM 8 TB/s, dense bf16
 * 2.5 PFLOP/s).  libgdr_roofline.so is a measurement aid and no part of the
 * path's boundary (gdr.h).
 *
 * Each entry point only enqueues one kernel on `stream` (a hipStream_t, NULL
 * for the default stream); the caller times it with events.  Buffers are
 * caller-owned device memory, 16-byte aligned.  Return value: 0 on success,
 * -1 for a bad argument (nothing launched), -3 if the launch failed.
 */
#ifndef GDR_ROOFLINE_H
#define GDR_ROOFLINE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * In-place read-modify-write stream: every 256-thread workgroup loads one
 * 64 KiB slab (16 x 16 bytes per lane, all loads issued first), multiplies it
 * by `scale` and stores it back -- the access pattern of the decode step.
 * bytes: a positive multiple of 65536.  nontemporal != 0 streams past the
 * last-level cache.  Traffic: 2 * bytes.
 */
int gdr_roofline_rmw(float* buf, size_t bytes, float scale, int nontemporal, void* stream);

/*
 * Read-only stream: every 256-thread workgroup sums one 64 KiB slab of `buf`
 * and writes the sum to sums[workgroup] (bytes / 65536 floats).  bytes: a
 * positive multiple of 65536.  Traffic: bytes (+ 4 bytes per 64 KiB).
 */
int gdr_roofline_read(const float* buf, size_t bytes, float* sums, void* stream);

/*
 * Dense bf16 matrix-core issue: `workgroups` workgroups of 256 threads, each
 * wave running `iters` rounds of 8 independent v_mfma_f32_16x16x32_bf16 (16
 * x 16 x 32 multiply-adds each); each wave writes one float of its
 * accumulators to out[global wave index] (workgroups * 4 floats).
 * FLOPs: workgroups * 4 * iters * 8 * 16384.  workgroups, iters > 0.
 */
int gdr_roofline_mfma(float* out, int workgroups, int iters, void* stream);

/*
 * Vector-ALU issue: `workgroups` workgroups of 256 threads, each thread
 * running `iters` rounds of 8 independent a = a * m + c chains with the
 * multiply and the add as separate fp32 instructions (16 VALU instructions
 * per wave per round, no dependency stalls); each wave writes one float to
 * out[global wave index] (workgroups * 4 floats).  Wave-level VALU
 * instructions: workgroups * 4 * iters * 16 (plus a few dozen per wave).
 * workgroups, iters > 0.
 */
int gdr_roofline_valu(float* out, int workgroups, int iters, void* stream);

/*
 * Exhaustive checks of the numeric behaviour that the conv front's bit-exact
 * contract (SiLU by exp32 and an IEEE division, then round to nearest even to
 * bf16; deepmagic page, architecture section: the kernel-4 causal conv and
 * SiLU in front of the recurrence) relies on, run over the fp32 bit patterns
 * first_bits .. first_bits + count - 1 (count <= 2^32, wrapping past
 * 0xffffffff).  *mismatches (zeroed by the caller) gains the number of
 * patterns that fail; *first_mismatch (set to 0xffffffff by the caller) is
 * lowered to the smallest failing pattern.
 *   silu_mid: the conv kernel's SiLU for |v| <= 80 (one residual correction
 *             of v * rcp(d)) equals the contract's SiLU (v / d with the IEEE
 *             division) bit for bit; patterns outside [-80, 80] and NaN are
 *             skipped
 *   bf16_rne: the hardware fp32 -> bf16 conversion equals round to nearest
 *             even on the bit pattern, and turns a NaN into a quiet NaN of
 *             the same sign
 */
int gdr_probe_silu_mid(uint32_t first_bits, unsigned long long count, unsigned long long* mismatches,
                       uint32_t* first_mismatch, void* stream);
int gdr_probe_bf16_rne(uint32_t first_bits, unsigned long long count, unsigned long long* mismatches,
                       uint32_t* first_mismatch, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDR_ROOFLINE_H */
