/*
 * lds_transpose.h - gfx950 LDS-to-register transpose microbenchmark
 * (liblds_transpose.so, built beside libattn.so; a measurement tool, not part
 * of the attention ABI).
 *
 * It repeats, on MI355X, the comparison of Rao et al., "Scheduling Data to
 * Compute: Hierarchical Data Pipelining for LLM Training on AMD GPUs",
 * section 4.3.2, Table 10: how fast each way of bringing a transposed matrix
 * operand from LDS into registers runs, against a plain 16-byte row load
 * (section 3.1.2, Tables 4 and 5 describe the ways).
 */
#ifndef MI355_LDS_TRANSPOSE_H
#define MI355_LDS_TRANSPOSE_H

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Time one method over `reps` launches and keep the fastest.
 *   method        0 ds_read_b128 of an operand that needs no transpose
 *                 1 ds_read_b64_tr_b16 (the transpose load), two per operand
 *                 2 eight 16-bit loads, one per row
 *                 3 ds_read_b128 of a row, then an 8 x 8 transpose across lanes
 *                   with three XOR shuffle stages
 *   blocks        workgroups of 256 threads; each wave loads `iters` x 8 operands
 *                 of 16 bytes per lane from a 64 x 64 bf16 tile in LDS
 *   ms_out        host pointer: the fastest launch's duration in milliseconds
 *   operand_out   device pointer, 16-byte aligned, 2048 words: the operand
 *                 lane l loads at position p (0..7, the eight 16-row x 32-column
 *                 blocks one loop iteration reads) in words 4(64p + l) .. +3
 *                 (methods 1-3 give the same values)
 *   checksum_out  device pointer, blocks * 256 words: per-thread XOR of every
 *                 loaded word (keeps the loads live)
 *   stream        hipStream_t as void*; the call synchronises on it
 * Returns 0 on success, 1 for an unknown method, 2 for bad sizes or pointers,
 * 3 for a HIP error. Every launch writes the same outputs.
 */
int lds_transpose_bench(int method, int blocks, int iters, int reps, float* ms_out,
                        unsigned int* operand_out, unsigned int* checksum_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MI355_LDS_TRANSPOSE_H */
