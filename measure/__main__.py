import sys

from measure import main

sys.exit(main(sys.argv))
