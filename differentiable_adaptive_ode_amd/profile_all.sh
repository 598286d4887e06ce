#!/bin/bash
# Profiles of the benchmark's calls on the current kernels: for each workload
# and mode, a kernel trace, the HBM byte counters (with a calibration copy),
# the issued floating-point instruction counters, instruction and stall
# counters, then profiling.py's summary into $OUT/profiles (copied into
# profiles/ by hand once read).  On a machine with the GPU:
#   [OUT=dir] bash differentiable_adaptive_ode_amd/profile_all.sh [TAG MODE WORKLOAD N ...]
# OUT defaults to profile_runs/ at the repository root.
set -u
cd "$(dirname "$0")/.." || exit 1
OUT=${OUT:-profile_runs}
export TMPDIR=/tmp
mkdir -p "$OUT/profiles"

prof() {  # TAG MODE WORKLOAD N
  local TAG=$1 MODE=$2 WL=$3 N=$4
  local B="python3 bench.py --mode $MODE --workload $WL --no-cpu-baseline --configs 0"
  local CT="rocprofv3 --kernel-trace --stats -f csv -d $OUT/prof_${TAG}_trace -o run -- $B --steps 5 --warmup 1"
  local CF="rocprofv3 --pmc FETCH_SIZE -f csv -d $OUT/prof_${TAG}_fetch -o run -- $B --steps 3 --warmup 1 --copy-calibration 256"
  local CW="rocprofv3 --pmc WRITE_SIZE -f csv -d $OUT/prof_${TAG}_write -o run -- $B --steps 3 --warmup 1 --copy-calibration 256"
  local CFL="rocprofv3 --pmc SQ_INSTS_VALU_ADD_F64 SQ_INSTS_VALU_MUL_F64 SQ_INSTS_VALU_FMA_F64 SQ_INSTS_VALU_TRANS_F64 SQ_INSTS_VALU_FLOPS_FP64 SQ_INSTS_VALU_FLOPS_FP32 SQ_INSTS_VALU_MFMA_MOPS_F32 SQ_WAVES -f csv -d $OUT/prof_${TAG}_flops -o run -- $B --steps 3 --warmup 1 --copy-calibration 256"
  local CS="rocprofv3 --pmc SQ_WAVES SQ_INSTS_VALU SQ_INSTS_SALU SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_INSTS_MFMA SQ_INSTS_VALU_FMA_F64 SQ_INSTS_LDS -f csv -d $OUT/prof_${TAG}_sq -o run -- $B --steps 3 --warmup 1 --copy-calibration 256"
  local CST="rocprofv3 --pmc SQ_WAVE_CYCLES SQ_WAIT_INST_ANY SQ_WAIT_ANY SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_ANY SQ_THREAD_CYCLES_VALU SQ_WAVES -f csv -d $OUT/prof_${TAG}_stall -o run -- $B --steps 3 --warmup 1"
  echo "== $TAG trace"
  timeout -k 10 240 $CT > $OUT/prof_${TAG}_trace.log 2>&1 || { echo "trace rc=$?"; tail -5 $OUT/prof_${TAG}_trace.log; return 1; }
  echo "== $TAG fetch"
  timeout -s KILL 240 $CF > $OUT/prof_${TAG}_fetch.log 2>&1 || { echo "fetch rc=$?"; tail -5 $OUT/prof_${TAG}_fetch.log; return 1; }
  echo "== $TAG write"
  timeout -s KILL 240 $CW > $OUT/prof_${TAG}_write.log 2>&1 || { echo "write rc=$?"; tail -5 $OUT/prof_${TAG}_write.log; return 1; }
  echo "== $TAG flops"
  timeout -s KILL 240 $CFL > $OUT/prof_${TAG}_flops.log 2>&1 || { echo "flops rc=$?"; tail -5 $OUT/prof_${TAG}_flops.log; return 1; }
  echo "== $TAG sq"
  timeout -s KILL 240 $CS > $OUT/prof_${TAG}_sq.log 2>&1 || { echo "sq rc=$?"; tail -5 $OUT/prof_${TAG}_sq.log; return 1; }
  echo "== $TAG stall"
  timeout -s KILL 240 $CST > $OUT/prof_${TAG}_stall.log 2>&1 || { echo "stall rc=$?"; tail -5 $OUT/prof_${TAG}_stall.log; return 1; }
  python3 -m differentiable_adaptive_ode_amd.profiling summarize --workload "$TAG" --n "$N" \
    --trace $OUT/prof_${TAG}_trace --fetch $OUT/prof_${TAG}_fetch \
    --write $OUT/prof_${TAG}_write --cmd-trace "$CT" --cmd-fetch "$CF" --cmd-write "$CW" \
    --flops $OUT/prof_${TAG}_flops --cmd-flops "$CFL" --sq $OUT/prof_${TAG}_sq \
    --cmd-sq "$CS" --stall $OUT/prof_${TAG}_stall --cmd-stall "$CST" --out $OUT/profiles
}

if [ $# -ge 4 ]; then
  while [ $# -ge 4 ]; do prof "$1" "$2" "$3" "$4" || exit 1; shift 4; done
  exit 0
fi
for spec in "loghalo gradient loghalo 1048576" "lorenz63 gradient lorenz63 65536" \
            "lotka_volterra gradient lotka_volterra 256" "mlp gradient mlp 16384" \
            "robertson gradient robertson 262144"; do
  prof $spec || exit 1
done
echo "profiles done"
