"""CPU oracle of the Token Recycling step -- test infrastructure only.

Only tests/, the smoke check and the CPU-baseline leg of the benchmark may
import this package.  It shares no code with the HIP library."""
