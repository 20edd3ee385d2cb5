"""CPU oracle of the selection-resolution step.  TEST INFRASTRUCTURE ONLY:
only the tests, the smoke check and the benchmark's CPU-baseline leg may
import it; the GPU library and its binding never do."""
